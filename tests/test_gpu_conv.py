"""Per-shard conv on the GPU against the oracle (small volumes, full oracle).

Covers every matrix-core instance (2D 64->64 k3, 3D 32->32 k3 on a 2x2x2
grid, 3D 16->16 k5, 2D 256->256 k3), the fp32 direct kernel and bf16 shapes
without a matrix-core instance; ragged tails against every tile shape;
batch 2; bias; the identity and shift kernels (bit-exact); and the method's
invariant that the sharded output equals the GPU's own unsharded output bit
for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from halo_sharded_conv_amd.layer import ShardedConvGN
from helpers import TOL, bits_equal, direct_cases, oracle_forward, rel_err, say, small_cases

pytestmark = pytest.mark.gpu

CASES = {**small_cases(), **direct_cases()}


def run(wl, x, w, bias=None, **kw):
    layer = ShardedConvGN(wl, **kw)
    layer.set_weight(w, bias)
    layer.load_input(x)
    layer.step()
    torch.cuda.synchronize()
    return layer


@pytest.mark.parametrize("name", list(CASES))
def test_conv_matches_oracle(name):
    wl = CASES[name]
    say(f"conv vs oracle: {name} spatial={wl.spatial} shards={wl.shards} N={wl.batch}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    bias = np.random.default_rng(5).uniform(-0.5, 0.5, wl.cout).astype(np.float32)
    layer = run(wl, x, w, bias)
    y_ref, _ = oracle_forward(wl, x, w, bias)
    err = rel_err(layer.y_host(), y_ref)
    say(f"  max|err|/rms(y) = {err:.3e}  (tolerance {TOL[wl.dtype]:.0e})")
    assert err <= TOL[wl.dtype]


@pytest.mark.parametrize("name", list(CASES))
def test_sharded_equals_unsharded_bitwise(name):
    wl = CASES[name]
    say(f"sharded == unsharded: {name}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    a = run(wl, x, w)
    b = run(wl.unsharded(), x, w)
    # one shard runs deeper jobs (several steps per job) than the sharded
    # layout does: hold it to the oracle too, so equal bits mean right bits
    y_ref, _ = oracle_forward(wl, x, w, None)
    err = rel_err(b.y_host(), y_ref)
    say(f"  unsharded max|err|/rms(y) = {err:.3e}")
    assert err <= TOL[wl.dtype]
    assert bits_equal(a.y_host(), b.y_host())
    assert bits_equal(a.z_host(), b.z_host())


@pytest.mark.parametrize("name", ["vol32_full", "img64_small", "vol32_grid", "vol16k5", "grid256_small",
                                  "img_c5to12_k3"])
def test_identity_kernel_exact(name):
    wl = CASES[name]
    if wl.cin != wl.cout:
        wl = dataclasses.replace(wl, cout=wl.cin, groups=1)
    say(f"identity kernel: {name}")
    x = synth.make_input(wl)
    k = wl.ksize
    w = np.zeros(wl.w_shape, np.float32)
    for o in range(wl.cout):
        w[(o, o) + (k // 2,) * wl.ndim] = 1.0
    if wl.dtype == "bf16":
        w = synth.f32_to_bf16_bits(w)
    layer = run(wl, x, w)
    want = oracle.widen(x, wl.dtype).astype(np.float32)
    assert bits_equal(layer.y_host(), want)


@pytest.mark.parametrize("name", ["vol32_full", "img64_b2", "vol32_grid", "vol16k5", "vol16k5_b2", "grid256_small"])
def test_shift_kernel_exact(name):
    """One-hot kernel at a corner tap: y[i] = x[i + t - p] with zeros entering
    at the global faces; crosses every shard seam, face, edge and corner."""
    wl = CASES[name]
    if wl.cin != wl.cout:
        wl = dataclasses.replace(wl, cout=wl.cin, groups=1)
    x = synth.make_input(wl)
    k, p, d = wl.ksize, wl.ksize // 2, wl.ndim
    for t in [(0,) * d, (k - 1,) * d, tuple([k - 1] + [0] * (d - 1))]:
        say(f"shift kernel {name} tap {t}")
        w = np.zeros(wl.w_shape, np.float32)
        for o in range(wl.cout):
            w[(o, (o + 1) % wl.cin) + t] = 1.0
        if wl.dtype == "bf16":
            w = synth.f32_to_bf16_bits(w)
        layer = run(wl, x, w)
        xf = oracle.widen(x, wl.dtype).astype(np.float32)
        xf = np.roll(xf, -1, axis=-1)                          # output o <- input o+1
        want = np.zeros_like(xf)
        src, dst = [slice(None)], [slice(None)]
        for a in range(d):
            sh = t[a] - p
            n = wl.spatial[a]
            src.append(slice(max(0, sh), min(n, n + sh)))
            dst.append(slice(max(0, -sh), min(n, n - sh)))
        want[tuple(dst)] = xf[tuple(src)]
        assert bits_equal(layer.y_host(), want)


def test_conv_plan_independent_of_uneven_splits():
    """Several different shard plans of one volume give identical bits."""
    base = CASES["img64_small"]
    x, w = synth.make_input(base), synth.make_weight(base)
    ref = run(base.unsharded(), x, w).y_host()
    for shards in [((1, 36), (70,)), ((18, 19), (33, 37)), ((5, 5, 5, 22), (16, 54))]:
        say(f"plan {shards}")
        got = run(base.with_shards(shards), x, w).y_host()
        assert bits_equal(got, ref)


@pytest.mark.parametrize("name", list(CASES))
def test_packed_entry_point_gives_the_same_bits(name):
    """st_conv_sharded_packed on weights packed once by st_conv_pack_weights
    writes the same y and max |y| as st_conv_sharded, which packs the raw
    weights into its workspace on every call."""
    import halo_sharded_conv_amd as hsc
    wl = CASES[name]
    say(f"packed entry point == raw-weight entry point: {name}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    layer = run(wl, x, w)
    packed = torch.zeros(hsc.st_conv_weight_bytes(wl.ndim, wl.cin, wl.cout, wl.ksize, wl.dtype), dtype=torch.uint8,
                         device="cuda")
    hsc.st_conv_pack_weights(wl.ndim, wl.cin, wl.cout, wl.ksize, wl.dtype, layer.w_raw, packed)
    ys = [torch.full_like(y, float("nan")) for y in layer.y_bufs]
    ymax = torch.full_like(layer.ymax, -1)
    hsc.st_conv_sharded_packed(layer.in_plan, layer.x_bufs, packed, None, wl.cout, wl.ksize, ys, ymax, wl.groups)
    torch.cuda.synchronize()
    for a, b in zip(layer.y_bufs, ys):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(layer.ymax, ymax)
