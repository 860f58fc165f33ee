"""GroupNorm backward on the GPU against the oracle.

The backward call reads the forward pass's y and (mean, rstd) and an upstream
gradient dz, and writes dy, dgamma and dbeta.  Checks: all three against the
oracle's group_norm_backward (fp64, pinned on the CPU) evaluated on the GPU's
own y, within the fp32 tolerance; sharded equal to unsharded bit for bit;
a caller-supplied max |dz| giving the same bits as the computed one; dy
aliasing dz; a zero upstream gradient giving exact zeros; dy written straight
into the input-gradient layer's padded bf16 (or fp32) shards equal to the
rounded same-layout dy, margins untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from halo_sharded_conv_amd.layer import ShardedConvGN
from helpers import bits_equal, direct_cases, rel_err, say, small_cases

pytestmark = pytest.mark.gpu

CASES = {**small_cases(), **direct_cases()}
TOL_BWD = 1e-5      # every step of the backward pass is fp32 arithmetic


def forward_backward(wl, x, w, dz, gamma=None, beta=None, dzmax=None, alias_dy=False):
    layer = ShardedConvGN(wl)
    layer.set_weight(w)
    layer.set_affine(gamma, beta)
    layer.load_input(x)
    layer.step()
    layer.alloc_backward()
    layer.load_upstream_grad(dz)
    dm = None
    if dzmax is not None:
        dm = torch.from_numpy(dzmax.view(np.int32)).cuda()
    layer.norm_backward(dzmax=dm, dy_bufs=layer.dz_bufs if alias_dy else None)
    torch.cuda.synchronize()
    return layer


def host_dzmax(wl, dz):
    g = dz.reshape(wl.batch, -1, wl.groups, wl.cout // wl.groups)
    return np.abs(g).max(axis=(1, 3)).astype(np.float32)


@pytest.mark.parametrize("name", list(CASES))
def test_gn_backward_matches_oracle(name):
    wl = CASES[name]
    say(f"groupnorm backward vs oracle: {name} spatial={wl.spatial} shards={wl.shards} N={wl.batch}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    gamma, beta = synth.make_affine(wl, seed=13)
    dz = synth.make_upstream_grad(wl, seed=21)
    layer = forward_backward(wl, x, w, dz, gamma, beta)
    y = layer.y_host().astype(np.float64)
    dy_ref, dg_ref, db_ref = oracle.group_norm_backward(y, dz, wl.groups, wl.eps, gamma)
    e_dy = rel_err(layer.gather(layer.dy_bufs), dy_ref)
    e_dg = rel_err(layer.dgamma.cpu().numpy(), dg_ref)
    e_db = rel_err(layer.dbeta.cpu().numpy(), db_ref)
    say(f"  max|err|/rms: dy {e_dy:.2e} dgamma {e_dg:.2e} dbeta {e_db:.2e} (tolerance {TOL_BWD:.0e})")
    assert e_dy <= TOL_BWD and e_dg <= TOL_BWD and e_db <= TOL_BWD


@pytest.mark.parametrize("name", ["vol32_full", "vol32_b2", "img64_small", "img64_b2", "vol32_grid",
                                  "vol16k5", "grid256_small", "img_c5to12_k3", "vol_c3to4_k5"])
def test_gn_backward_sharded_equals_unsharded_bitwise(name):
    wl = CASES[name]
    say(f"groupnorm backward sharded == unsharded: {name}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    gamma, beta = synth.make_affine(wl, seed=17)
    dz = synth.make_upstream_grad(wl, seed=23)
    a = forward_backward(wl, x, w, dz, gamma, beta)
    b = forward_backward(wl.unsharded(), x, w, dz, gamma, beta)
    assert bits_equal(a.y_host(), b.y_host())
    assert bits_equal(a.gather(a.dy_bufs), b.gather(b.dy_bufs))
    assert bits_equal(a.dgamma.cpu().numpy(), b.dgamma.cpu().numpy())
    assert bits_equal(a.dbeta.cpu().numpy(), b.dbeta.cpu().numpy())


@pytest.mark.parametrize("name", ["img64_small", "vol32_grid", "img_c5to12_k3"])
def test_gn_backward_given_dzmax_and_aliasing(name):
    """A caller-supplied max |dz| and dy written over dz give the same bits."""
    wl = CASES[name]
    say(f"groupnorm backward, given max|dz| and dy over dz: {name}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    dz = synth.make_upstream_grad(wl, seed=29)
    a = forward_backward(wl, x, w, dz)
    b = forward_backward(wl, x, w, dz, dzmax=host_dzmax(wl, dz), alias_dy=True)
    assert bits_equal(a.gather(a.dy_bufs), b.gather(b.dz_bufs))
    assert bits_equal(a.dgamma.cpu().numpy(), b.dgamma.cpu().numpy())
    assert bits_equal(a.dbeta.cpu().numpy(), b.dbeta.cpu().numpy())


def test_gn_backward_zero_gradient():
    wl = CASES["img64_small"]
    x, w = synth.make_input(wl), synth.make_weight(wl)
    dz = np.zeros((wl.batch, *wl.spatial, wl.cout), np.float32)
    layer = forward_backward(wl, x, w, dz)
    assert not np.any(layer.gather(layer.dy_bufs))
    assert not np.any(layer.dgamma.cpu().numpy()) and not np.any(layer.dbeta.cpu().numpy())


@pytest.mark.parametrize("name", ["vol32_full", "img64_small", "img64_b2", "vol32_grid", "vol16k5",
                                  "grid256_small"])
def test_gn_backward_into_padded_input_gradient_shards(name):
    """dy written straight into the input-gradient layer's halo-padded shards
    (bf16 rounded to nearest even, or fp32): interiors equal the same-layout
    fp32 dy (rounded on the host), margins are not touched."""
    from halo_sharded_conv_amd.layer import dgrad_config
    wl = CASES[name]
    say(f"groupnorm backward into padded shards: {name}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    gamma, beta = synth.make_affine(wl, seed=19)
    dz = synth.make_upstream_grad(wl, seed=37)
    layer = forward_backward(wl, x, w, dz, gamma, beta)
    want = layer.gather(layer.dy_bufs)
    bwd = ShardedConvGN(dgrad_config(wl))
    for t in bwd.x_bufs:
        t.fill_(0x3F7B if t.dtype == torch.int16 else 0.625)   # sentinel margins
    layer.norm_backward(dy_bufs=bwd.x_bufs, dy_plan=bwd.in_plan)
    torch.cuda.synchronize()
    h = wl.ksize // 2
    for i in range(bwd.S):
        pad = bwd.padded_host(i)
        inner = tuple([slice(None)] + [slice(h, h + e) for e in bwd.info[i]["extent"]] + [slice(None)])
        part = want[bwd._global_slices(i)]
        expect = synth.f32_to_bf16_bits(part) if wl.dtype == "bf16" else part
        assert bits_equal(pad[inner], expect)
        mask = np.ones(pad.shape, bool)
        mask[inner] = False
        sentinel = np.uint16(0x3F7B) if wl.dtype == "bf16" else np.float32(0.625)
        assert np.all(pad[mask] == sentinel)
