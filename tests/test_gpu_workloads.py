"""All five workloads at full size, in the launch configuration the benchmark
times (sharded plan, fused max, separate z buffers).

  * y and z element by element against the oracle, streamed one slab of the
    outermost axis at a time (oracle.conv_same_slabbed, fp64): the whole
    tensor for the fp32 volume, the 2048^2 image, the 256^3 volume and the
    1024 x 1792 grid; for the 512^3 k5 volume (8.6 TFLOP of fp64 work in
    full) every depth plane of its thinnest shard plus the planes within the
    halo width of every other seam, each plane whole.  z from the oracle's y
    with the oracle's full-size per-group mean/variance stored in
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


def checked_rows(wl):
    """Row ranges of the outermost axis compared against the oracle: all of
    them, except on the 512^3 volume, where the thinnest shard's planes and
    the halo-width planes on both sides of every other seam are taken."""
    if wl.name != "vol512_c16_k5_bf16":
        return [(0, wl.spatial[0])]
    sizes = wl.shards[0]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(int)
    t = int(np.argmin(sizes))
    rows = set(range(off[t], off[t + 1]))
    for b in off[1:-1]:
        rows |= set(range(b - wl.halo, b + wl.halo))
    rows = sorted(rows)
    ranges, start = [], rows[0]
    for a, b in zip(rows, rows[1:] + [None]):
        if b != a + 1:
            ranges.append((start, a + 1))
            start = b
    return ranges


def streamed_errors(wl, layer, x, w, g, ranges):
    """max |gpu - oracle| / rms over the given row ranges, for y and z."""
    wf = oracle.widen(w, wl.dtype)
    ey = ez = 0.0
    n = 0
    slab = max(1, min(64, (1 << 22) // (int(np.prod(wl.spatial[1:])) * wl.cout)))
    for lo, hi in ranges:
        for s0, y_ref in oracle.conv_same_slabbed(x, wl.dtype, wf, None, slab=slab, start=lo, stop=hi):
            s1 = s0 + y_ref.shape[1]
            z_ref = oracle.group_norm_apply(y_ref, wl.groups, g["mean"], g["var"], wl.eps)
            ey = max(ey, float(np.max(np.abs(layer.gather_rows(layer.y_bufs, s0, s1) - y_ref))))
            ez = max(ez, float(np.max(np.abs(layer.gather_rows(layer.z_bufs, s0, s1) - z_ref))))
            n += y_ref.size
    return ey / g["rms_y"], ez / g["rms_z"], n


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
    ranges = checked_rows(wl)
    say(f"  oracle over rows {ranges}")
    ey, ez, n = streamed_errors(wl, layer, x, w, g, ranges)
    total = wl.batch * int(np.prod(wl.spatial)) * wl.cout
    say(f"  {n} of {total} outputs: max|err|/rms y {ey:.3e}  z {ez:.3e}  (tolerance {TOL[wl.dtype]:.0e})")
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


def test_checked_planes_cover_the_512_volume_seams():
    wl = synth.workload("vol512_c16_k5_bf16")
    ranges = checked_rows(wl)
    rows = {r for lo, hi in ranges for r in range(lo, hi)}
    off = np.cumsum(wl.shards[0])[:-1]
    for b in off:
        assert set(range(b - wl.halo, b + wl.halo)) <= rows
    assert len(rows) >= min(wl.shards[0])
