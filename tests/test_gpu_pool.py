"""Shape-changing sharded op on the GPU: 'valid' pooling with the output
sharding shapes derived by the library.

Tolerances: fp32 outputs 1e-5 of rms; bf16 outputs are one round-to-nearest
of the fp32 result, so each element is held to half a bf16 ulp (at most
2^-8 of its magnitude) plus 1e-6 of rms for the fp32 sum.

Input shards are halo-padded by ksize - 1 and exchanged (pack + unpack), then
st_pool_sharded writes every shard's owned outputs into the plan that
st_plan_pooled derived.  Checks: the derived shard sizes against the
oracle's pooled_shard_sizes; max pooling bit for bit against the oracle;
average pooling within the bound of the output type; sharded equal to unsharded bit for bit; output margins
untouched.
"""
import numpy as np
import pytest
import torch

import halo_sharded_conv_amd as hsc
import oracle
import synth
from helpers import TOL, bits_equal, rel_err, say, small_cases

pytestmark = pytest.mark.gpu

CASES = small_cases()


def global_slices(plan, i):
    inf = plan.shard_info(i)
    return tuple([slice(None)] + [slice(o, o + e) for o, e in zip(inf["offset"], inf["extent"])])


def interior(plan, t, i):
    inf = plan.shard_info(i)
    v = t.view(plan.padded_shape(i))
    return v[tuple([slice(None)] + [slice(h, h + e) for h, e in zip(plan.halo, inf["extent"])] + [slice(None)])]


def run_pool(wl, x, k, s, mode, out_dtype=None, sentinel=None):
    d = wl.ndim
    tdt = torch.float32 if wl.dtype == "f32" else torch.int16
    p = hsc.st_plan_shards(d, wl.batch, wl.cin, wl.spatial, wl.shards, [k - 1] * d, wl.dtype)
    bufs = [torch.zeros(p.shard_info(i)["elems"], dtype=tdt, device="cuda") for i in range(p.num_shards)]
    xs = x.view(np.int16) if x.dtype == np.uint16 else x
    for i in range(p.num_shards):
        interior(p, bufs[i], i).copy_(torch.from_numpy(np.ascontiguousarray(xs[global_slices(p, i)])))
    msg = torch.zeros(max(16, p.msg_bytes), dtype=torch.uint8, device="cuda")
    hsc.st_halo_pack(p, bufs, msg)
    hsc.st_halo_unpack(p, msg, bufs, True)
    q = hsc.st_plan_pooled(p, k, s, out_halo=[1] * d, out_dtype=out_dtype)
    odt = torch.float32 if q.dtype == hsc.ST_F32 else torch.int16
    outs = [torch.empty(q.shard_info(i)["elems"], dtype=odt, device="cuda") for i in range(q.num_shards)]
    for t in outs:
        t.fill_(sentinel if sentinel is not None else 0)
    hsc.st_pool_sharded(p, bufs, k, s, mode, q, outs)
    torch.cuda.synchronize()
    shape = (wl.batch, *[sum(a) for a in q.shards], wl.cin)
    got = np.empty(shape, np.float32 if q.dtype == hsc.ST_F32 else np.uint16)
    for i in range(q.num_shards):
        v = interior(q, outs[i], i).cpu().numpy()
        got[global_slices(q, i)] = v.view(np.uint16) if q.dtype != hsc.ST_F32 else v
    return p, q, got, outs


SPECS = [("img64_small", 2, 2, "avg", None), ("img64_small", 2, 2, "max", None), ("img64_small", 3, 2, "avg", "f32"),
         ("img64_b2", 2, 2, "avg", None), ("vol32_grid", 2, 2, "avg", None), ("vol32_grid", 2, 2, "max", None),
         ("vol32_grid", 3, 2, "max", None), ("vol32_grid", 3, 2, "avg", "f32"), ("vol32_full", 2, 2, "avg", None),
         ("vol32_full", 3, 3, "max", None), ("grid256_small", 2, 2, "avg", None), ("vol16k5", 2, 1, "avg", None)]


@pytest.mark.parametrize("name,k,s,mode,odt", SPECS)
def test_pool_matches_oracle(name, k, s, mode, odt):
    wl = CASES[name]
    say(f"pool vs oracle: {name} k={k} s={s} {mode} out={odt or wl.dtype} shards={wl.shards}")
    x = synth.make_input(wl)
    p, q, got, _ = run_pool(wl, x, k, s, mode, odt)
    for a in range(wl.ndim):
        assert list(q.shards[a]) == oracle.pooled_shard_sizes(p.shards[a], k, s)
    want = oracle.pool_valid(oracle.widen(x, wl.dtype), k, s, mode)
    out_bf16 = q.dtype == hsc.ST_BF16
    g = oracle.widen(got, "bf16") if out_bf16 else got.astype(np.float64)
    if mode == "max":
        assert np.array_equal(g, want)
    elif out_bf16:
        # one rounding of the fp32 average to bf16: at most half an ulp, which
        # is <= 2^-8 |value| for an 8-bit significand (plus the fp32 sum)
        rms = float(np.sqrt(np.mean(want * want)))
        excess = np.abs(g - want) - (2.0 ** -8 * np.abs(want) + 1e-6 * rms)
        say(f"  max|err|/rms = {rel_err(g, want):.2e}; worst excess over the bf16 rounding bound {excess.max():.2e}")
        assert excess.max() <= 0.0
    else:
        err = rel_err(g, want)
        say(f"  max|err|/rms = {err:.2e} (tolerance {TOL['f32']:.0e})")
        assert err <= TOL["f32"]


@pytest.mark.parametrize("name,k,s,mode", [("img64_small", 2, 2, "avg"), ("vol32_grid", 3, 2, "avg"),
                                           ("vol32_full", 2, 2, "max"), ("grid256_small", 3, 2, "avg")])
def test_pool_sharded_equals_unsharded_and_margins_untouched(name, k, s, mode):
    wl = CASES[name]
    say(f"pool sharded == unsharded: {name} k={k} s={s} {mode}")
    x = synth.make_input(wl)
    sentinel = 0x3F7B if wl.dtype == "bf16" else 0.625
    _, q, a, outs = run_pool(wl, x, k, s, mode, sentinel=sentinel)
    _, _, b, _ = run_pool(wl.unsharded(), x, k, s, mode)
    assert bits_equal(a, b)
    for i in range(q.num_shards):
        v = outs[i].view(q.padded_shape(i)).cpu().numpy()
        mask = np.ones(v.shape, bool)
        inf = q.shard_info(i)
        mask[tuple([slice(None)] + [slice(1, 1 + e) for e in inf["extent"]] + [slice(None)])] = False
        assert np.all(v[mask] == (np.int16(sentinel) if wl.dtype == "bf16" else np.float32(sentinel)))
