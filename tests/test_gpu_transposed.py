"""Transposed (upsampling) conv on the GPU with the output sharding shapes
derived by the library.

Input shards are halo-padded by ksize/2 and exchanged, then
st_conv_transposed_sharded writes every shard's outputs [a*s, (a+e)*s) into
the plan st_plan_transposed derived.  Checks: derived shard sizes are the
input's times the stride; x against oracle.conv_transposed (plus the bias)
within the fp32 tolerance (bf16 inputs widen exactly, products and sums are
fp32); sharded equal to unsharded bit for bit; the adjoint identity with the
GPU's own strided conv.
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
TOL_TRANSPOSED = 1e-5      # fp32 products and accumulation


def make_w(wl, cx, seed):
    """W [Cy][Cx][k..k] with Cy the input's channels (the strided conv's
    outputs), in the layer's operand type: float32, or bf16 bit patterns
    (uint16) rounded from the float32 draws."""
    r = np.random.default_rng(seed)
    w = r.uniform(-1, 1, size=(wl.cin, cx) + (wl.ksize,) * wl.ndim).astype(np.float32)
    return synth.f32_to_bf16_bits(w) if wl.dtype == "bf16" else w


def gather_plan(q, outs, batch):
    got = np.empty((batch, *[sum(a) for a in q.shards], q.channels), np.float32)
    for i in range(q.num_shards):
        inf = q.shard_info(i)
        got[tuple([slice(None)] + [slice(o, o + e) for o, e in zip(inf["offset"], inf["extent"])])] = \
            outs[i].view(q.padded_shape(i)).cpu().numpy()
    return got


def run_transposed(wl, y, w, bias, s):
    layer = ShardedConvGN(wl)                     # padded input shards with halo ksize // 2
    layer.load_input(y)
    layer.exchange()
    cx = w.shape[1]
    q = hsc.st_plan_transposed(layer.in_plan, wl.ksize, s, cx)
    outs = [torch.full((q.shard_info(i)["elems"],), 7.0, dtype=torch.float32, device="cuda")
            for i in range(q.num_shards)]
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).cuda()
    ws = dev_workspace(hsc.st_conv_transposed_workspace_bytes(layer.in_plan, cx, wl.ksize))
    # the raw weight bits go to the library, which widens and reorders them
    hsc.st_conv_transposed_sharded(layer.in_plan, layer.x_bufs, dev_raw(w), b, wl.ksize, s, q, outs, ws)
    torch.cuda.synchronize()
    return layer, q, gather_plan(q, outs, wl.batch)


SPECS = [("img64_small", 2), ("img64_b2", 2), ("vol32_grid", 2), ("vol16k5", 2), ("vol32_full", 2),
         ("grid256_small", 2), ("img_c5to12_k3", 2), ("vol_c3to4_k5", 3), ("vol32_b2", 3), ("img64_small", 1),
         ("img_c5to12_k3", 4), ("img_c64to48", 2),
         ("img64_small", 4), ("vol32_grid", 3)]     # matrix-core path with tapless phases; 27 phases in 3D


@pytest.mark.parametrize("name,s", SPECS)
def test_transposed_matches_oracle(name, s):
    wl = CASES[name]
    say(f"transposed conv vs oracle: {name} s={s} shards={wl.shards}")
    y = synth.make_input(wl)
    w = make_w(wl, wl.cout, seed=41 + s)
    bias = np.random.default_rng(5).uniform(-1, 1, wl.cout).astype(np.float32)
    layer, q, got = run_transposed(wl, y, w, bias, s)
    for a in range(wl.ndim):
        assert list(q.shards[a]) == [e * s for e in wl.shards[a]]
    want = oracle.conv_transposed(oracle.widen(y, wl.dtype), oracle.widen(w, wl.dtype), s) + bias
    err = rel_err(got, want)
    say(f"  max|err|/rms = {err:.2e} (tolerance {TOL_TRANSPOSED:.0e})")
    assert err <= TOL_TRANSPOSED


@pytest.mark.parametrize("name,s", [("img64_small", 2), ("vol32_grid", 2), ("vol16k5", 2), ("img_c5to12_k3", 3)])
def test_transposed_sharded_equals_unsharded(name, s):
    wl = CASES[name]
    say(f"transposed conv sharded == unsharded: {name} s={s}")
    y = synth.make_input(wl)
    w = make_w(wl, wl.cout, seed=43)
    _, _, a = run_transposed(wl, y, w, None, s)
    _, _, b = run_transposed(wl.unsharded(), y, w, None, s)
    assert bits_equal(a, b)


@pytest.mark.parametrize("name", ["img64_small", "vol32_grid"])
def test_transposed_is_adjoint_of_strided_on_gpu(name):
    """<strided(x, W), y> = <x, transposed(y, W)> with both sides computed on
    the GPU (fp64 dot products on the host), x of the transposed output's
    extent and sharding."""
    wl = CASES[name]
    s = 2
    say(f"transposed conv adjoint of strided conv: {name}")
    y = synth.make_input(wl)
    w = make_w(wl, wl.cout, seed=47)
    _, q, xt = run_transposed(wl, y, w, None, s)
    # x: fp32 input of the strided conv with the transposed output's plan, halo ksize // 2
    xw = dataclasses.replace(wl, name=wl.name + "_adjoint", spatial=tuple(sum(a) for a in q.shards),
                             shards=tuple(tuple(a) for a in q.shards), cin=wl.cout, cout=wl.cin, groups=1,
                             dtype="f32")
    xl = ShardedConvGN(xw)
    x = np.random.default_rng(53).standard_normal((wl.batch, *xw.spatial, wl.cout)).astype(np.float32)
    xl.load_input(x)
    xl.exchange()
    sq = hsc.st_plan_strided(xl.in_plan, wl.ksize, s, wl.cin)
    outs = [torch.empty(sq.shard_info(i)["elems"], dtype=torch.float32, device="cuda") for i in range(sq.num_shards)]
    # the strided conv from x (Cx channels) to y (Cy) takes W in conv order
    # [out = Cy][in = Cx]: the same array; this fp32 layer gets its fp32
    # values (torch widens the bf16 patterns exactly)
    wd = dev_raw(w)
    wd = wd.view(torch.bfloat16).float() if wl.dtype == "bf16" else wd
    ws = dev_workspace(hsc.st_conv_strided_workspace_bytes(xl.in_plan, wl.cin, wl.ksize))
    hsc.st_conv_strided_sharded(xl.in_plan, xl.x_bufs, wd, None, wl.ksize, s, sq, outs, ws)
    torch.cuda.synchronize()
    ys = gather_plan(sq, outs, wl.batch)
    yw = oracle.widen(y, wl.dtype)
    lhs = float(np.sum(ys.astype(np.float64) * yw))
    rhs = float(np.sum(x.astype(np.float64) * xt))
    scale = float(np.sum(np.abs(ys.astype(np.float64) * yw)))
    say(f"  <strided x, y> = {lhs:.6e}, <x, transposed y> = {rhs:.6e}")
    assert abs(lhs - rhs) <= 1e-5 * scale
