"""All five workloads at full size, in the launch configuration the benchmark
times (sharded plan, fused max, separate z buffers).

  * y and z at ~4k sampled positions (every shard seam, face and corner plus
    random cells) against the oracle: y by direct fp64 dot products, z from
    those with the oracle's full-size per-group mean/variance stored in
    tests/golden/ (written by tests/golden/make_golden.py, oracle only);
  * the GPU's (mean, rstd) against the same statistics;
  * the sharded y and z equal the GPU's own unsharded run bit for bit,
    compared over the whole tensors on the device.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from halo_sharded_conv_amd.layer import ShardedConvGN
from helpers import TOL, say, torch_bits_equal

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
from make_golden import load as load_golden  # noqa: E402

pytestmark = pytest.mark.gpu


def sampled_errors(wl, layer, x, w, g, count=4096):
    pos = synth.sample_positions(wl, count, seed=1)
    wf = oracle.widen(w, wl.dtype)
    y_ref = oracle.conv_at(x, wl.dtype, wf, None, pos)
    z_ref = np.empty_like(y_ref)
    for n in range(wl.batch):
        rows = pos[:, 0] == n
        z_ref[rows] = oracle.group_norm_apply(y_ref[rows][None], wl.groups, g["mean"][n:n + 1],
                                              g["var"][n:n + 1], wl.eps)[0]
    y_gpu = layer.at(layer.y_bufs, pos)
    z_gpu = layer.at(layer.z_bufs, pos)
    ey = float(np.max(np.abs(y_gpu - y_ref))) / g["rms_y"]
    ez = float(np.max(np.abs(z_gpu - z_ref))) / g["rms_z"]
    return ey, ez, len(pos)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_full_size(name):
    wl = synth.workload(name)
    g = load_golden(name)
    assert g["shards"] == [list(s) for s in wl.shards]
    say(f"workload {name}: generating inputs")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    say("  sharded run")
    layer = ShardedConvGN(wl)
    layer.set_weight(w)
    layer.load_input(x)
    layer.step()
    torch.cuda.synchronize()
    ey, ez, npos = sampled_errors(wl, layer, x, w, g)
    say(f"  sampled {npos} positions: max|err|/rms y {ey:.3e}  z {ez:.3e}  (tolerance {TOL[wl.dtype]:.0e})")
    assert ey <= TOL[wl.dtype] and ez <= TOL[wl.dtype]
    st = layer.gn_state()["stats"]
    scale = np.sqrt(g["var"] + wl.eps)
    dm = float(np.max(np.abs(st[..., 0] - g["mean"]) / scale))
    dr = float(np.max(np.abs(st[..., 1] * scale - 1.0)))
    say(f"  stats: |dmean|/sigma {dm:.2e}  |drstd|/rstd {dr:.2e}")
    assert dm < 1e-5 and dr < 1e-5

    say("  unsharded run")
    ref = ShardedConvGN(wl.unsharded())
    ref.set_weight(w)
    ref.load_input(x)
    del x
    ref.step()
    torch.cuda.synchronize()
    assert torch.equal(ref.ymax, layer.ymax)
    yu, zu = ref.out_view(ref.y_bufs, 0), ref.out_view(ref.z_bufs, 0)
    for s in range(layer.S):
        sl = layer._global_slices(s)
        assert torch_bits_equal(layer.out_view(layer.y_bufs, s), yu[sl].contiguous()), f"y shard {s}"
        assert torch_bits_equal(layer.out_view(layer.z_bufs, s), zu[sl].contiguous()), f"z shard {s}"
    say("  sharded == unsharded bitwise")
