"""Split-statistics GroupNorm on the GPU.

z against the oracle's unsharded conv + GroupNorm (fp64); the per-shard
partial sums against an exact integer recomputation from the GPU's own y;
the fused-max and separate-max paths giving the same bits; a zero-variance
group normalising to beta; random affine parameters; z aliasing y.
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


def run(wl, x, w, bias=None, gamma=None, beta=None, **kw):
    layer = ShardedConvGN(wl, **kw)
    layer.set_weight(w, bias)
    layer.set_affine(gamma, beta)
    layer.load_input(x)
    layer.step()
    torch.cuda.synchronize()
    return layer


@pytest.mark.parametrize("name", list(CASES))
def test_groupnorm_matches_oracle(name):
    wl = CASES[name]
    say(f"groupnorm vs oracle: {name}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    gamma, beta = synth.make_affine(wl, seed=11)
    layer = run(wl, x, w, None, gamma, beta)
    _, z_ref = oracle_forward(wl, x, w, None, gamma, beta)
    err = rel_err(layer.z_host(), z_ref)
    say(f"  max|err|/rms(z) = {err:.3e}  (tolerance {TOL[wl.dtype]:.0e})")
    assert err <= TOL[wl.dtype]
    # (mean, rstd) against the oracle's two-pass moments
    y_ref, _ = oracle_forward(wl, x, w)
    mean, var = oracle.group_moments(y_ref, wl.groups)
    st = layer.gn_state()["stats"]
    scale = np.sqrt(var + wl.eps)
    assert np.max(np.abs(st[..., 0] - mean) / scale) < 1e-5
    assert np.max(np.abs(st[..., 1] * scale - 1.0)) < 1e-5


@pytest.mark.parametrize("name", list(CASES))
def test_partial_sums_are_exact(name):
    """Per-shard sums equal the exact integers sum(rint(y * 2^e1)) and
    sum(rint(y^2 * 2^e2)) recomputed on the host from the GPU's own y."""
    wl = CASES[name]
    say(f"exact partials: {name}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    layer = run(wl, x, w)
    state = layer.gn_state()
    G, gs = wl.groups, wl.cout // wl.groups
    ymax = layer.ymax.cpu().numpy().view(np.float32).reshape(wl.batch, G)
    y_all = layer.y_host().astype(np.float64)
    assert np.array_equal(ymax, np.abs(y_all).reshape(wl.batch, -1, G, gs).max(axis=(1, 3)).astype(np.float32))
    M = gs * int(np.prod(wl.spatial))
    L = int(M).bit_length()
    for s in range(layer.S):
        ys = layer.out_view(layer.y_bufs, s).cpu().numpy().astype(np.float64)
        for n in range(wl.batch):
            part = ys[n].reshape(-1, G, gs)
            for g in range(G):
                m = float(ymax[n, g])
                e = int(np.frexp(m)[1]) if m > 0 else 0
                e1, e2 = (52 - L - e, 52 - L - 2 * e) if m > 0 else (0, 0)
                assert tuple(state["scales"][n, g]) == (e1, e2)
                v = part[:, g, :]
                q1 = np.rint(v * 2.0 ** e1).astype(np.int64).sum()
                q2 = np.rint((v * v) * 2.0 ** e2).astype(np.int64).sum()
                assert state["partials"][s, n, g, 0] == float(q1)
                assert state["partials"][s, n, g, 1] == float(q2)
                assert abs(int(q1)) < 2 ** 52 and abs(int(q2)) < 2 ** 52


@pytest.mark.parametrize("name", ["vol32_b2", "img64_small", "vol16k5", "img_c5to12_k3"])
def test_unfused_max_gives_same_bits(name):
    wl = CASES[name]
    say(f"unfused max: {name}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    a = run(wl, x, w)
    b = run(wl, x, w, fuse_max=False)
    assert bits_equal(a.z_host(), b.z_host())


@pytest.mark.parametrize("name,groups", [("img64_small", 64), ("img64_small", 16), ("img64_b2", 1),
                                         ("vol32_grid", 32), ("vol32_grid", 16), ("vol32_grid", 4),
                                         ("vol16k5", 16), ("vol16k5", 8), ("grid256_small", 128)])
def test_fused_max_every_group_size(name, groups):
    """The conv epilogue keeps its running max|y| per 1, 2 or 4 channels,
    whichever divides the group size; every granularity must give the same
    per-group maxima (and so the same GroupNorm bits) as the separate pass."""
    wl = dataclasses.replace(CASES[name], groups=groups)
    say(f"fused max: {name} groups={groups}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    a = run(wl, x, w)
    b = run(wl, x, w, fuse_max=False)
    y = a.y_host()
    want = np.abs(y.reshape(wl.batch, -1, groups, wl.cout // groups)).max(axis=(1, 3))
    assert np.array_equal(a.ymax.cpu().numpy().view(np.float32).reshape(wl.batch, groups), want)
    assert np.array_equal(a.gn_state()["scales"], b.gn_state()["scales"])
    assert bits_equal(a.z_host(), b.z_host())


@pytest.mark.parametrize("name", ["img64_small", "vol32_full"])
def test_alias_z_onto_y(name):
    wl = CASES[name]
    x, w = synth.make_input(wl), synth.make_weight(wl)
    a = run(wl, x, w)
    b = run(wl, x, w, alias_z=True)
    assert bits_equal(a.z_host(), b.z_host())


@pytest.mark.parametrize("name", ["img64_small", "vol32_full", "img_c5to12_k3"])
def test_zero_variance_group_gives_beta(name):
    wl = CASES[name]
    say(f"zero-variance group: {name}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    gs = wl.cout // wl.groups
    if wl.dtype == "bf16":
        wf = oracle.widen(w, "bf16").astype(np.float32)
    else:
        wf = w.copy()
    wf[:gs] = 0.0                                        # group 0: y = bias (constant)
    bias = np.full(wl.cout, 0.75, np.float32)
    w2 = synth.f32_to_bf16_bits(wf) if wl.dtype == "bf16" else wf
    gamma, beta = synth.make_affine(wl, seed=3)
    layer = run(wl, x, w2, bias, gamma, beta)
    z = layer.z_host()
    assert np.array_equal(z[..., :gs], np.broadcast_to(beta[:gs], z[..., :gs].shape))
    _, z_ref = oracle_forward(wl, x, w2, bias, gamma, beta)
    assert rel_err(z, z_ref) <= TOL[wl.dtype]


def test_all_zero_output():
    wl = CASES["img64_small"]
    x = synth.make_input(wl)
    w = np.zeros(wl.w_shape, np.uint16)
    gamma, beta = synth.make_affine(wl, seed=4)
    layer = run(wl, x, w, None, gamma, beta)
    assert np.array_equal(layer.y_host(), np.zeros_like(layer.y_host()))
    z = layer.z_host()
    assert np.array_equal(z, np.broadcast_to(beta, z.shape))


@pytest.mark.parametrize("name", ["vol32_b2", "img64_b2", "vol16k5", "img_c5to12_k3", "grid256_small", "img_c6to10_k3"])
def test_combined_apply_matches_three_calls(name):
    """st_groupnorm_sharded folds the combine into the apply's prologue when
    the per-lane coefficient path applies; z and the stored (mean, rstd) must
    be the same bits as partials, combine and apply called one by one."""
    wl = CASES[name]
    say(f"combine folded into apply vs three calls: {name}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    gamma, beta = synth.make_affine(wl, seed=5)
    a = run(wl, x, w, None, gamma, beta)
    b = run(wl, x, w, None, gamma, beta)
    for zb in b.z_bufs:
        zb.fill_(float("nan"))
    b.norm_partials()
    b.norm_combine()
    b.norm_apply()
    torch.cuda.synchronize()
    assert bits_equal(a.z_host(), b.z_host())
    assert bits_equal(a.gn_state()["stats"], b.gn_state()["stats"])
