"""Weight gradient of the sharded conv on the GPU against the oracle.

The forward layer's padded x (after its halo exchange) and a gradient dy at
y (held in the input-gradient layer's shard buffers, the layout the backward
pass already has) go to st_conv_wgrad.  Checks: dw against the oracle's
conv_same_wgrad (fp64, pinned on the CPU) within the forward tolerance of
the operand type, for every small case (matrix-core instances and the
direct kernel); the same plan twice gives the same bits; sharded and
unsharded runs both meet the tolerance (their fp32 accumulations group the
positions differently, so they are not compared bit for bit).
"""
import numpy as np
import pytest
import torch

import halo_sharded_conv_amd as hsc
import oracle
import synth
from halo_sharded_conv_amd.layer import ShardedConvGN, dgrad_config
from helpers import TOL, bits_equal, direct_cases, rel_err, say, small_cases

pytestmark = pytest.mark.gpu

CASES = {**small_cases(), **direct_cases()}


def run_wgrad(wl, x, dy):
    fwd = ShardedConvGN(wl)
    fwd.load_input(x)
    fwd.exchange()
    bwd = ShardedConvGN(dgrad_config(wl))
    bwd.load_input(dy)
    dw = torch.empty(wl.cout * wl.cin * wl.taps, dtype=torch.float32, device="cuda")
    ws = torch.empty(hsc.st_conv_wgrad_workspace_bytes(fwd.in_plan, wl.cout, wl.ksize), dtype=torch.uint8,
                     device="cuda")
    hsc.st_conv_wgrad(fwd.in_plan, fwd.x_bufs, bwd.in_plan, bwd.x_bufs, wl.ksize, dw, ws)
    torch.cuda.synchronize()
    return dw.cpu().numpy().reshape(wl.w_shape)


def inputs(wl, seed_shift=0):
    x = synth.make_input(wl)
    dy = synth.make_input(dgrad_config(wl))
    return x, dy


@pytest.mark.parametrize("name", list(CASES))
def test_wgrad_matches_oracle(name):
    wl = CASES[name]
    say(f"wgrad vs oracle: {name} spatial={wl.spatial} shards={wl.shards} N={wl.batch}")
    x, dy = inputs(wl)
    got = run_wgrad(wl, x, dy)
    want = oracle.conv_same_wgrad(oracle.widen(x, wl.dtype), oracle.widen(dy, wl.dtype), wl.ksize)
    err = rel_err(got, want)
    say(f"  max|err|/rms(dw) = {err:.3e}  (tolerance {TOL[wl.dtype]:.0e})")
    assert err <= TOL[wl.dtype]


@pytest.mark.parametrize("name", ["img64_small", "vol32_grid", "vol16k5_b2", "grid256_small", "vol32_b2",
                                  "img_c5to12_k3"])
def test_wgrad_deterministic_and_plan_independent_within_tolerance(name):
    wl = CASES[name]
    say(f"wgrad repeatability and unsharded run: {name}")
    x, dy = inputs(wl)
    a = run_wgrad(wl, x, dy)
    b = run_wgrad(wl, x, dy)
    assert bits_equal(a, b)
    c = run_wgrad(wl.unsharded(), x, dy)
    want = oracle.conv_same_wgrad(oracle.widen(x, wl.dtype), oracle.widen(dy, wl.dtype), wl.ksize)
    assert rel_err(c, want) <= TOL[wl.dtype]
    assert rel_err(a, c) <= TOL[wl.dtype]


def test_wgrad_image_tall_shards():
    """The 64-channel image layer on 4 uneven shards of a 300 x 520 image:
    many rows per partition, ragged W chunks."""
    base = synth.WORKLOADS["img2048_c64_k3_bf16"]
    wl = synth.small_variant(base, (300, 520), ((90, 61, 77, 72), (520,)), name_suffix="tall")
    say(f"wgrad vs oracle: {wl.name}")
    x, dy = inputs(wl)
    got = run_wgrad(wl, x, dy)
    want = oracle.conv_same_wgrad(oracle.widen(x, wl.dtype), oracle.widen(dy, wl.dtype), wl.ksize)
    err = rel_err(got, want)
    say(f"  max|err|/rms(dw) = {err:.3e}")
    assert err <= TOL[wl.dtype]
