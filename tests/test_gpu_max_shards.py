"""Plans at the API's shard limit (ST_MAX_SHARDS = 64) on the GPU.

Every kernel takes its per-shard table by value; these cases fill all 64
entries: a 4 x 4 x 4 grid of 3D shards (the 32-channel and 16-channel k5
layers) and an 8 x 8 grid of image shards.  Through every entry point: halo
exchange (padded shards bit for bit against the oracle's), conv + GroupNorm
and the GroupNorm backward (sharded == unsharded bit for bit, oracle
tolerance), the weight gradient (oracle tolerance), and the strided conv, the
transposed conv and pooling (derived sizes, sharded == unsharded bit for bit,
oracle tolerance).
"""
import numpy as np
import pytest
import torch

import halo_sharded_conv_amd as hsc
import oracle
import synth
from helpers import TOL, bits_equal, dev_workspace, oracle_forward, rel_err, say
from test_gpu_random_plans import _gather, _shape_ops, forward

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
CASES = {
    "vol32_4x4x4": synth.small_variant(W["vol256_c32_k3_bf16"], (12, 13, 14),
                                       ((3, 3, 3, 3), (3, 4, 3, 3), (4, 3, 3, 4))),
    "vol16k5_4x4x4": synth.small_variant(W["vol512_c16_k5_bf16"], (9, 10, 11),
                                         ((2, 2, 2, 3), (2, 2, 3, 3), (3, 2, 2, 4))),
    "img64_8x8": synth.small_variant(W["img2048_c64_k3_bf16"], (20, 33),
                                     ((2, 3, 2, 3, 2, 3, 2, 3), (4, 4, 5, 4, 4, 4, 4, 4))),
}


@pytest.mark.parametrize("name", list(CASES))
def test_max_shards_forward_and_halo(name):
    wl = CASES[name]
    assert wl.num_shards == hsc.ST_MAX_SHARDS
    say(f"64 shards, forward + GroupNorm backward: {name} shards={wl.shards}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    gamma, beta = synth.make_affine(wl, seed=3)
    dz = synth.make_upstream_grad(wl, seed=9)
    a = forward(wl, x, w, gamma, beta, dz)
    # the exchanged padded shards, bit for bit against the oracle's
    for i, idx in enumerate(oracle.shard_grid(wl.shards)):
        want = oracle.padded_shard(x, wl.shards, idx, wl.halo)
        assert bits_equal(a.padded_host(i), want), f"padded shard {i} {idx}"
    b = forward(wl.unsharded(), x, w, gamma, beta, dz)
    assert bits_equal(a.y_host(), b.y_host()) and bits_equal(a.z_host(), b.z_host())
    assert bits_equal(a.gather(a.dy_bufs), b.gather(b.dy_bufs))
    assert bits_equal(a.dgamma.cpu().numpy(), b.dgamma.cpu().numpy())
    y_ref, z_ref = oracle_forward(wl, x, w, None, gamma, beta)
    ey, ez = rel_err(a.y_host(), y_ref), rel_err(a.z_host(), z_ref)
    say(f"  max|err|/rms y {ey:.2e} z {ez:.2e}")
    assert ey <= TOL[wl.dtype] and ez <= TOL[wl.dtype]
    # weight gradient over all 64 shards
    dy = a.gather(a.dy_bufs)
    dyb = synth.f32_to_bf16_bits(dy)
    from halo_sharded_conv_amd.layer import ShardedConvGN, dgrad_config
    g = ShardedConvGN(dgrad_config(wl))
    g.load_input(dyb)
    dw = torch.empty(wl.cout * wl.cin * wl.taps, dtype=torch.float32, device="cuda")
    ws = dev_workspace(hsc.st_conv_wgrad_workspace_bytes(a.in_plan, wl.cout, wl.ksize))
    hsc.st_conv_wgrad(a.in_plan, a.x_bufs, g.in_plan, g.x_bufs, wl.ksize, dw, ws)
    torch.cuda.synchronize()
    want = oracle.conv_same_wgrad(oracle.widen(x, wl.dtype), oracle.widen(dyb, wl.dtype), wl.ksize)
    e = rel_err(dw.cpu().numpy().reshape(want.shape), want)
    say(f"  weight gradient max|err|/rms {e:.2e}")
    assert e <= TOL[wl.dtype]


@pytest.mark.parametrize("name", list(CASES))
def test_max_shards_shape_changing_ops(name):
    wl = CASES[name]
    say(f"64 shards, strided / transposed / pooling: {name}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    bias = np.random.default_rng(4).uniform(-1, 1, wl.cout).astype(np.float32)
    a = _shape_ops(wl, x, w, bias)
    u = _shape_ops(wl.unsharded(), x, w, bias)
    xf, wf = oracle.widen(x, wl.dtype), oracle.widen(w, wl.dtype)
    q, outs = a["strided"]
    assert q.num_shards == hsc.ST_MAX_SHARDS
    for ax in range(wl.ndim):
        assert list(q.shards[ax]) == oracle.strided_shard_sizes(wl.shards[ax], wl.ksize, 2)
    got = _gather(q, outs, wl.batch)
    assert bits_equal(got, _gather(*u["strided"], wl.batch))
    assert rel_err(got, oracle.conv_strided(xf, wf, 2, bias)) <= 1e-5
    q, outs, wtr = a["transposed"]
    got = _gather(q, outs, wl.batch)
    assert bits_equal(got, _gather(*u["transposed"][:2], wl.batch))
    assert rel_err(got, oracle.conv_transposed(xf, oracle.widen(wtr, wl.dtype), 2) + bias) <= 1e-5
    q, outs = a["pool"]
    for ax in range(wl.ndim):
        assert list(q.shards[ax]) == oracle.pooled_shard_sizes(wl.shards[ax], 2, 2)
    got = _gather(q, outs, wl.batch, np.uint16)
    assert bits_equal(got, _gather(*u["pool"], wl.batch, np.uint16))
    want = oracle.pool_valid(xf, 2, 2, "avg")
    g = oracle.widen(got, "bf16")
    rms = float(np.sqrt(np.mean(want * want)))
    assert np.all(np.abs(g - want) <= 2.0 ** -8 * np.abs(want) + 1e-6 * rms)
