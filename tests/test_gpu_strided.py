"""Strided (downsampling) conv on the GPU with the output sharding shapes
derived by the library.

Input shards are halo-padded by ksize/2 and exchanged, then
st_conv_strided_sharded writes every shard's owned outputs into the plan
st_plan_strided derived.  Checks: derived shard sizes against the oracle's
strided_shard_sizes; y against oracle.conv_strided within the fp32
tolerance (bf16 operands multiply exactly in fp32, so 1e-5 holds for them
too); sharded equal to unsharded bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import halo_sharded_conv_amd as hsc
import oracle
import synth
from halo_sharded_conv_amd.layer import ShardedConvGN
from helpers import bits_equal, dev_raw, dev_workspace, direct_cases, rel_err, say, small_cases

pytestmark = pytest.mark.gpu

CASES = {**small_cases(), **direct_cases()}
# 64 -> 48 channels: a 32-row tile and a half-filled one on the matrix cores
CASES["img_c64to48"] = dataclasses.replace(CASES["img64_small"], name="img_c64to48", cout=48, groups=4)
TOL_STRIDED = 1e-5      # fp32 accumulation of exact products


def run_strided(wl, x, w, bias, s):
    layer = ShardedConvGN(wl)                     # padded input shards with halo ksize // 2
    layer.load_input(x)
    layer.exchange()
    q = hsc.st_plan_strided(layer.in_plan, wl.ksize, s, wl.cout)
    outs = [torch.empty(q.shard_info(i)["elems"], dtype=torch.float32, device="cuda") for i in range(q.num_shards)]
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).cuda()
    ws = dev_workspace(hsc.st_conv_strided_workspace_bytes(layer.in_plan, wl.cout, wl.ksize))
    # the synth bits go to the library as they are: it widens and reorders them
    hsc.st_conv_strided_sharded(layer.in_plan, layer.x_bufs, dev_raw(w), b, wl.ksize, s, q, outs, ws)
    torch.cuda.synchronize()
    got = np.empty((wl.batch, *[sum(a) for a in q.shards], wl.cout), np.float32)
    for i in range(q.num_shards):
        inf = q.shard_info(i)
        got[tuple([slice(None)] + [slice(o, o + e) for o, e in zip(inf["offset"], inf["extent"])])] = \
            outs[i].view(q.padded_shape(i)).cpu().numpy()
    return layer, q, got


SPECS = [("img64_small", 2), ("img64_b2", 2), ("vol32_grid", 2), ("vol16k5", 2), ("vol32_full", 2),
         ("grid256_small", 2), ("img_c5to12_k3", 2), ("vol_c3to4_k5", 3), ("vol32_b2", 3), ("img_c64to48", 2),
         ("img64_small", 1), ("vol16k5", 1)]      # stride 1: the 'same' conv


@pytest.mark.parametrize("name,s", SPECS)
def test_strided_matches_oracle(name, s):
    wl = CASES[name]
    say(f"strided conv vs oracle: {name} s={s} shards={wl.shards}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    bias = np.random.default_rng(3).uniform(-1, 1, wl.cout).astype(np.float32)
    layer, q, got = run_strided(wl, x, w, bias, s)
    for a in range(wl.ndim):
        assert list(q.shards[a]) == oracle.strided_shard_sizes(wl.shards[a], wl.ksize, s)
    want = oracle.conv_strided(oracle.widen(x, wl.dtype), oracle.widen(w, wl.dtype), s, bias)
    if s == 1:      # stride 1 is the 'same' conv of the forward layer
        assert got.shape == want.shape == x.shape[:-1] + (wl.cout,)
    err = rel_err(got, want)
    say(f"  max|err|/rms = {err:.2e} (tolerance {TOL_STRIDED:.0e})")
    assert err <= TOL_STRIDED


@pytest.mark.parametrize("name,s", [("img64_small", 2), ("vol32_grid", 2), ("vol16k5", 2), ("img_c5to12_k3", 3)])
def test_strided_sharded_equals_unsharded(name, s):
    wl = CASES[name]
    say(f"strided conv sharded == unsharded: {name} s={s}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    _, _, a = run_strided(wl, x, w, None, s)
    _, _, b = run_strided(wl.unsharded(), x, w, None, s)
    assert bits_equal(a, b)
