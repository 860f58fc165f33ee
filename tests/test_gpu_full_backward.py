"""The backward step and the shape-changing ops at full size, in the launch
configuration the benchmark times, on the image workload (1x64x2048x2048
bf16 on four uneven H shards) and on the 256^3 volume (1x32x256^3 bf16 on a
2 x 2 x 2 grid of uneven shards: faces, edges and corners).

Backward chain as `bench.py --pass backward` runs it: the sharded forward
step, GroupNorm backward writing bf16 dy straight into the input-gradient
layer's padded shards, their halo exchange, the input-gradient conv and the
weight gradient.  Each stage is checked against the fp64 oracle over the
whole tensor, fed the GPU's own inputs to that stage (y, and the bf16 dy
read back), so each error belongs to one stage:
  * dy, dgamma, dbeta vs oracle.group_norm_backward (1e-5 of rms for the
    fp32 dy before rounding; the padded bf16 dy equals its rounding);
  * dx vs oracle.conv_same_dgrad, dw vs oracle.conv_same_wgrad (1e-2);
  * the 2x average pooling of the input vs oracle.pool_valid (bf16 rounding
    bound) and the derived output shard sizes vs oracle.pooled_shard_sizes;
  * the stride-2 conv of the input vs oracle.conv_strided over the whole
    output (1e-5), with the derived shard sizes;
  * the stride-2 transposed conv from half resolution (every shard halved)
    vs oracle.conv_transposed over the whole output (1e-5).
"""
import numpy as np
import pytest
import torch

import halo_sharded_conv_amd as hsc
import oracle
import synth
from halo_sharded_conv_amd.layer import ShardedConvGN, dgrad_config
from helpers import TOL, bits_equal, dev_raw, dev_workspace, rel_err, say

pytestmark = pytest.mark.gpu

NAMES = ["img2048_c64_k3_bf16", "vol256_c32_k3_bf16"]


@pytest.mark.parametrize("NAME", NAMES)
def test_full_size_backward_chain(NAME):
    wl = synth.workload(NAME)
    say(f"full-size backward {NAME}: inputs")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    dz = synth.make_upstream_grad(wl, seed=31)
    fwd = ShardedConvGN(wl)
    fwd.set_weight(w)
    fwd.load_input(x)
    fwd.step()
    fwd.alloc_backward()
    fwd.load_upstream_grad(dz)
    bwd = ShardedConvGN(dgrad_config(wl))
    bwd.set_weight_dgrad(w)
    say("  GPU: GroupNorm backward (fp32 and into the padded bf16 shards), exchange, dgrad, wgrad")
    fwd.norm_backward()                                            # fp32 dy in y's layout
    fwd.norm_backward(dy_bufs=bwd.x_bufs, dy_plan=bwd.in_plan)     # bf16 dy, padded
    bwd.exchange()
    bwd.conv()
    dw = torch.empty(wl.cout * wl.cin * wl.taps, dtype=torch.float32, device="cuda")
    ws = torch.empty(hsc.st_conv_wgrad_workspace_bytes(fwd.in_plan, wl.cout, wl.ksize), dtype=torch.uint8,
                     device="cuda")
    hsc.st_conv_wgrad(fwd.in_plan, fwd.x_bufs, bwd.in_plan, bwd.x_bufs, wl.ksize, dw, ws)
    torch.cuda.synchronize()

    y = fwd.y_host()
    dy32 = fwd.gather(fwd.dy_bufs)
    say("  oracle: GroupNorm backward")
    dy_ref, dg_ref, db_ref = oracle.group_norm_backward(y.astype(np.float64), dz, wl.groups, wl.eps)
    e = (rel_err(dy32, dy_ref), rel_err(fwd.dgamma.cpu().numpy(), dg_ref), rel_err(fwd.dbeta.cpu().numpy(), db_ref))
    say(f"  max|err|/rms dy {e[0]:.2e} dgamma {e[1]:.2e} dbeta {e[2]:.2e} (tolerance 1e-5)")
    assert max(e) <= 1e-5
    del dy_ref
    dyb = np.empty((wl.batch, *wl.spatial, wl.cout), np.uint16)
    for i in range(bwd.S):
        dyb[bwd._global_slices(i)] = bwd.interior_view(i).cpu().numpy().view(np.uint16)
    assert bits_equal(dyb, synth.f32_to_bf16_bits(dy32))
    del dy32
    dyf = oracle.widen(dyb, "bf16")
    del dyb
    say("  oracle: input gradient")
    dx_ref = oracle.conv_same_dgrad(dyf, oracle.widen(w, wl.dtype))
    e_dx = rel_err(bwd.y_host(), dx_ref)
    del dx_ref
    say("  oracle: weight gradient")
    dw_ref = oracle.conv_same_wgrad(oracle.widen(x, wl.dtype), dyf, wl.ksize)
    e_dw = rel_err(dw.cpu().numpy().reshape(dw_ref.shape), dw_ref)
    say(f"  max|err|/rms dx {e_dx:.2e} dw {e_dw:.2e} (tolerance {TOL[wl.dtype]:.0e})")
    assert e_dx <= TOL[wl.dtype] and e_dw <= TOL[wl.dtype]


@pytest.mark.parametrize("NAME", NAMES)
def test_full_size_pooling(NAME):
    wl = synth.workload(NAME)
    say(f"full-size 2x average pooling {NAME}")
    x = synth.make_input(wl)
    p = hsc.st_plan_shards(wl.ndim, wl.batch, wl.cin, wl.spatial, wl.shards, [1] * wl.ndim, wl.dtype)
    q = hsc.st_plan_pooled(p, 2, 2)
    for a in range(wl.ndim):
        assert list(q.shards[a]) == oracle.pooled_shard_sizes(wl.shards[a], 2, 2)
    layer = ShardedConvGN(wl)               # its input plan has the same shards and halo 1
    layer.load_input(x)
    layer.exchange()
    outs = [torch.empty(q.shard_info(i)["elems"], dtype=torch.int16, device="cuda") for i in range(q.num_shards)]
    hsc.st_pool_sharded(layer.in_plan, layer.x_bufs, 2, 2, "avg", q, outs)
    torch.cuda.synchronize()
    got = np.empty((wl.batch, *[sum(a) for a in q.shards], wl.cin), np.uint16)
    for i in range(q.num_shards):
        inf = q.shard_info(i)
        got[tuple([slice(None)] + [slice(o, o + e) for o, e in zip(inf["offset"], inf["extent"])])] = \
            outs[i].view(q.padded_shape(i)).cpu().numpy().view(np.uint16)
    want = oracle.pool_valid(oracle.widen(x, wl.dtype), 2, 2, "avg")
    g = oracle.widen(got, "bf16")
    rms = float(np.sqrt(np.mean(want * want)))
    excess = np.abs(g - want) - (2.0 ** -8 * np.abs(want) + 1e-6 * rms)
    say(f"  max|err|/rms {rel_err(g, want):.2e}; worst excess over the bf16 rounding bound {excess.max():.2e}")
    assert excess.max() <= 0.0


@pytest.mark.parametrize("NAME", NAMES)
def test_full_size_strided_conv(NAME):
    wl = synth.workload(NAME)
    say(f"full-size stride-2 conv {NAME}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    layer = ShardedConvGN(wl)
    layer.load_input(x)
    layer.exchange()
    q = hsc.st_plan_strided(layer.in_plan, wl.ksize, 2, wl.cout)
    for a in range(wl.ndim):
        assert list(q.shards[a]) == oracle.strided_shard_sizes(wl.shards[a], wl.ksize, 2)
    outs = [torch.empty(q.shard_info(i)["elems"], dtype=torch.float32, device="cuda") for i in range(q.num_shards)]
    ws = dev_workspace(hsc.st_conv_strided_workspace_bytes(layer.in_plan, wl.cout, wl.ksize))
    hsc.st_conv_strided_sharded(layer.in_plan, layer.x_bufs, dev_raw(w), None, wl.ksize, 2, q, outs, ws)
    torch.cuda.synchronize()
    got = np.empty((wl.batch, *[sum(a) for a in q.shards], wl.cout), np.float32)
    for i in range(q.num_shards):
        inf = q.shard_info(i)
        got[tuple([slice(None)] + [slice(o, o + e) for o, e in zip(inf["offset"], inf["extent"])])] = \
            outs[i].view(q.padded_shape(i)).cpu().numpy()
    want = oracle.conv_strided(oracle.widen(x, wl.dtype), oracle.widen(w, wl.dtype), 2)
    err = rel_err(got, want)
    say(f"  max|err|/rms {err:.2e} (tolerance 1e-5)")
    assert err <= 1e-5


def half_shards(sizes):
    """Per-axis shard sizes of a half-resolution input: every shard halved
    (rounded down), the last one taking the rest."""
    n = sum(sizes) // 2
    head = [e // 2 for e in sizes[:-1]]
    return tuple(head + [n - sum(head)])


@pytest.mark.parametrize("NAME", NAMES)
def test_full_size_transposed_conv(NAME):
    """The bench's upsampling workload: the layer at half resolution (every
    shard halved) up to full size (the image workload's sharding shapes; on
    the 256^3 grid, whose extents are odd, the halved shards times two),
    bias included, over the whole output."""
    import dataclasses
    wl_out = synth.workload(NAME)
    wl = dataclasses.replace(wl_out, name=wl_out.name + "_half", spatial=tuple(n // 2 for n in wl_out.spatial),
                             shards=tuple(half_shards(a) for a in wl_out.shards))
    say(f"full-size stride-2 transposed conv {wl.name} {wl.shards} -> {NAME}")
    y, w = synth.make_input(wl), synth.make_weight(wl)
    layer = ShardedConvGN(wl)
    layer.load_input(y)
    layer.exchange()
    q = hsc.st_plan_transposed(layer.in_plan, wl.ksize, 2, wl.cout)
    assert q.shards == tuple(tuple(2 * e for e in a) for a in wl.shards)
    wtr = np.ascontiguousarray(np.swapaxes(w, 0, 1))                # W [in = Cin][out = Cout][k..], raw bits
    bias = np.random.default_rng(7).uniform(-1, 1, wl.cout).astype(np.float32)
    outs = [torch.empty(q.shard_info(i)["elems"], dtype=torch.float32, device="cuda") for i in range(q.num_shards)]
    ws = dev_workspace(hsc.st_conv_transposed_workspace_bytes(layer.in_plan, wl.cout, wl.ksize))
    hsc.st_conv_transposed_sharded(layer.in_plan, layer.x_bufs, dev_raw(wtr), torch.from_numpy(bias).cuda(),
                                   wl.ksize, 2, q, outs, ws)
    torch.cuda.synchronize()
    got = np.empty((wl.batch, *[sum(a) for a in q.shards], wl.cout), np.float32)
    for i in range(q.num_shards):
        inf = q.shard_info(i)
        got[tuple([slice(None)] + [slice(o, o + e) for o, e in zip(inf["offset"], inf["extent"])])] = \
            outs[i].view(q.padded_shape(i)).cpu().numpy()
    del outs
    want = oracle.conv_transposed(oracle.widen(y, wl.dtype), oracle.widen(wtr, wl.dtype), 2) + bias
    err = rel_err(got, want)
    say(f"  max|err|/rms {err:.2e} (tolerance 1e-5)")
    assert err <= 1e-5
