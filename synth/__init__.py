"""Seeded synthetic workloads for the halo-sharded conv + GroupNorm layer.

This module is shared by the oracle side and the GPU side of every test and of
the benchmark.  It holds the workload table, the shard-size generator and the
input generators only: it performs none of the layer's arithmetic (no
convolution, no normalisation, no halo logic).

Provenance of the workloads: the ShardTensor summary pages ("Technical summary:
ShardTensor - domain parallelism for scientific machine learning", section 2
"Design principles") describe splitting the spatial axes of one sample into
uneven chunks ("sharding shapes") and exchanging halos so that convolution and
normalisation stay numerically consistent (section 2 "Implementation details",
"Communication").  The pages give no sizes for this layer; the five workloads
below are synthetic stand-ins.  The weather-grid workload takes the 1024 x 1792
CONUS grid and the 2-way activation split that section 4 ("StormScope") reports.

Layout of every array handed out here is channels-last: x is [N, *spatial, C].
Weights are [Cout, Cin, *taps] (PyTorch's logical order).
bf16 inputs are returned as uint16 bit patterns, rounded to nearest-even from
the float32 draws; the same bit patterns go to the GPU and to the oracle.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "BENCH_WORKLOAD", "workload", "shard_sizes",
    "f32_to_bf16_bits", "make_input", "make_weight", "make_affine",
    "sample_positions", "small_variant",
]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs must be finite.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("bf16 rounding of non-finite inputs is outside the workloads")
    b = a.view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def shard_sizes(total: int, parts: int, lo: int, hi: Optional[int],
                rng: np.random.Generator) -> list:
    """Draw an uneven split of `total` into `parts` sizes, each in [lo, hi].

    Uniform random composition by rejection: the `free = total - parts*lo`
    cells above the floor are cut at parts-1 sorted integer points drawn from
    [0, free]; redraw while a size exceeds `hi`.
    """
    free = total - parts * lo
    if free < 0:
        raise ValueError("total too small for the lower bound")
    if hi is not None and hi * parts < total:
        raise ValueError("upper bound too small for the total")
    if parts == 1:
        return [total]
    for _ in range(1_000_000):
        cuts = np.sort(rng.integers(0, free, size=parts - 1, endpoint=True))
        sizes = lo + np.diff(np.concatenate([[0], cuts, [free]]))
        if hi is None or int(sizes.max()) <= hi:
            return [int(s) for s in sizes]
    raise RuntimeError("rejection sampling did not meet the upper bound")


@dataclasses.dataclass(frozen=True)
class Workload:
    """One conv + GroupNorm layer over a domain-sharded volume."""
    name: str
    ndim: int                      # 2 or 3 spatial axes
    batch: int
    cin: int
    cout: int
    spatial: Tuple[int, ...]       # (H, W) or (D, H, W)
    ksize: int                     # odd cubic kernel, stride 1, 'same' zero padding
    groups: int
    eps: float
    dtype: str                     # "f32" or "bf16": operand type of the conv
    shards: Tuple[Tuple[int, ...], ...]   # per spatial axis: shard sizes, low index first
    x_seed: int
    w_seed: int
    x_kind: str = "normal"         # "normal" or "channel_affine"
    xc_seed: Optional[int] = None  # seed of per-channel (mu_c, sigma_c) for channel_affine

    @property
    def halo(self) -> int:
        return self.ksize // 2

    @property
    def taps(self) -> int:
        return self.ksize ** self.ndim

    @property
    def voxels(self) -> int:
        return self.batch * math.prod(self.spatial)

    @property
    def num_shards(self) -> int:
        return math.prod(len(s) for s in self.shards)

    @property
    def conv_flops(self) -> int:
        return 2 * self.voxels * self.cin * self.cout * self.taps

    @property
    def x_shape(self) -> Tuple[int, ...]:
        return (self.batch, *self.spatial, self.cin)

    @property
    def w_shape(self) -> Tuple[int, ...]:
        return (self.cout, self.cin) + (self.ksize,) * self.ndim

    def with_shards(self, shards) -> "Workload":
        return dataclasses.replace(self, shards=tuple(tuple(int(v) for v in s) for s in shards))

    def unsharded(self) -> "Workload":
        return self.with_shards([(n,) for n in self.spatial])


def _seeded(total, parts, lo, hi, seed):
    return tuple(shard_sizes(total, parts, lo, hi, np.random.default_rng(seed)))


def _seeded_axes(specs, seed):
    rng = np.random.default_rng(seed)
    return tuple(tuple(shard_sizes(t, p, lo, hi, rng)) for (t, p, lo, hi) in specs)


WORKLOADS = {
    # fp32 3D conv, 1x4x32^3, k3, depth split 17/15, GroupNorm(4).
    "vol32_c4to8_k3_fp32": Workload(
        "vol32_c4to8_k3_fp32", 3, 1, 4, 8, (32, 32, 32), 3, 4, 1e-5, "f32",
        ((17, 15), (32,), (32,)), 101, 201),
    # bf16 2D conv, 1x64x2048^2, k3, 4 uneven H shards >= 256 rows, GroupNorm(32).
    "img2048_c64_k3_bf16": Workload(
        "img2048_c64_k3_bf16", 2, 1, 64, 64, (2048, 2048), 3, 32, 1e-5, "bf16",
        (_seeded(2048, 4, 256, None, 302), (2048,)), 102, 202),
    # bf16 3D conv, 1x32x256^3, k3, 2x2x2 grid, each split 128 +-10%, GroupNorm(8).
    "vol256_c32_k3_bf16": Workload(
        "vol256_c32_k3_bf16", 3, 1, 32, 32, (256, 256, 256), 3, 8, 1e-5, "bf16",
        _seeded_axes([(256, 2, 116, 140)] * 3, 303), 103, 203),
    # bf16 3D wide stencil, 1x16x512^3, k5, 8 depth shards of 48..80, GroupNorm(4).
    "vol512_c16_k5_bf16": Workload(
        "vol512_c16_k5_bf16", 3, 1, 16, 16, (512, 512, 512), 5, 4, 1e-5, "bf16",
        (_seeded(512, 8, 48, 80, 304), (512,), (512,)), 104, 204),
    # bf16 2D weather grid 1x256x1024x1792, k3, W split 900/892, GroupNorm(32).
    "grid1024x1792_c256_k3_bf16": Workload(
        "grid1024x1792_c256_k3_bf16", 2, 1, 256, 256, (1024, 1792), 3, 32, 1e-5, "bf16",
        ((1024,), (900, 892)), 105, 205, x_kind="channel_affine", xc_seed=405),
}

# The workload the throughput figure is quoted on: the largest volume that
# one GPU holds, 1x16x512^3 with the 5^3 stencil (2^27 output voxels).
BENCH_WORKLOAD = "vol512_c16_k5_bf16"


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _channel_params(wl: Workload):
    rng = np.random.default_rng(wl.xc_seed)
    mu = rng.uniform(-2.0, 2.0, size=wl.cin).astype(np.float32)
    sigma = rng.uniform(0.1, 5.0, size=wl.cin).astype(np.float32)
    return mu, sigma


def make_input(wl: Workload) -> np.ndarray:
    """The input volume, channels-last [N, *spatial, Cin].

    Values are drawn from one numpy PCG64 stream seeded with `x_seed`, in
    memory order, one slab of the outermost spatial axis at a time (so the
    largest volume never exists in float32 at once).  fp32 workloads return
    float32; bf16 workloads return the uint16 bf16 patterns.
    """
    rng = np.random.default_rng(wl.x_seed)
    slab = wl.spatial[1:] + (wl.cin,)
    out_dtype = np.float32 if wl.dtype == "f32" else np.uint16
    out = np.empty(wl.x_shape, dtype=out_dtype)
    if wl.x_kind == "channel_affine":
        mu, sigma = _channel_params(wl)
    for n in range(wl.batch):
        for i in range(wl.spatial[0]):
            v = rng.standard_normal(size=slab, dtype=np.float32)
            if wl.x_kind == "channel_affine":
                v = mu + sigma * v
            out[n, i] = v if wl.dtype == "f32" else f32_to_bf16_bits(v)
    return out


def make_weight(wl: Workload) -> np.ndarray:
    """Weights [Cout, Cin, *taps] ~ U(-1/sqrt(fan_in), +1/sqrt(fan_in)).

    float32 for fp32 workloads, uint16 bf16 patterns otherwise.
    """
    rng = np.random.default_rng(wl.w_seed)
    a = 1.0 / math.sqrt(wl.cin * wl.taps)
    w = rng.uniform(-a, a, size=wl.w_shape).astype(np.float32)
    return w if wl.dtype == "f32" else f32_to_bf16_bits(w)


def make_affine(wl: Workload, seed: Optional[int] = None):
    """GroupNorm affine (gamma, beta) per output channel, float32.

    seed=None gives the identity (gamma=1, beta=0) used by the workloads;
    a seed gives gamma ~ U(0.5, 1.5), beta ~ U(-1, 1) for tests.
    """
    if seed is None:
        return np.ones(wl.cout, np.float32), np.zeros(wl.cout, np.float32)
    rng = np.random.default_rng(seed)
    gamma = rng.uniform(0.5, 1.5, size=wl.cout).astype(np.float32)
    beta = rng.uniform(-1.0, 1.0, size=wl.cout).astype(np.float32)
    return gamma, beta


def make_upstream_grad(wl: Workload, seed: int) -> np.ndarray:
    """A gradient arriving at the layer's output, channels-last
    [N, *spatial, Cout] float32 ~ N(0, 1), drawn in memory order from one
    PCG64 stream (one slab of the outermost axis at a time)."""
    rng = np.random.default_rng(seed)
    out = np.empty((wl.batch, *wl.spatial, wl.cout), np.float32)
    for n in range(wl.batch):
        for i in range(wl.spatial[0]):
            out[n, i] = rng.standard_normal(size=wl.spatial[1:] + (wl.cout,), dtype=np.float32)
    return out


def _boundaries(sizes: Sequence[int]):
    off = np.concatenate([[0], np.cumsum(sizes)])
    return [int(v) for v in off]


def sample_positions(wl: Workload, count: int, seed: int) -> np.ndarray:
    """Output positions [count', 1 + ndim] as (n, *spatial) for sampled checks.

    Contains every combination of {first, last} along each axis, cells on both
    sides of every shard seam (and the halo-width cells next to it), then
    uniform random positions up to `count` in total.
    """
    rng = np.random.default_rng(seed)
    h = wl.halo
    per_axis = []
    for ax, sizes in enumerate(wl.shards):
        n = wl.spatial[ax]
        pts = {0, n - 1}
        for b in _boundaries(sizes)[1:-1]:
            for d in range(-h - 1, h + 1):
                if 0 <= b + d < n:
                    pts.add(b + d)
        per_axis.append(sorted(pts))
    special = []
    for ax in range(wl.ndim):
        # seam/face cells on this axis, random coordinates on the others
        for v in per_axis[ax]:
            pos = [int(rng.integers(0, wl.batch))]
            for a2 in range(wl.ndim):
                pos.append(v if a2 == ax else int(rng.integers(0, wl.spatial[a2])))
            special.append(pos)
    # corners of the whole volume
    for corner in range(2 ** wl.ndim):
        pos = [wl.batch - 1]
        for a2 in range(wl.ndim):
            pos.append(wl.spatial[a2] - 1 if (corner >> a2) & 1 else 0)
        special.append(pos)
    rest = max(0, count - len(special))
    rnd = np.stack([rng.integers(0, wl.batch, size=rest)] +
                   [rng.integers(0, s, size=rest) for s in wl.spatial], axis=1)
    return np.concatenate([np.asarray(special, dtype=np.int64).reshape(-1, 1 + wl.ndim),
                           rnd.astype(np.int64)], axis=0)


def small_variant(wl: Workload, spatial: Sequence[int], shards, batch: int = 1,
                  name_suffix: str = "small") -> Workload:
    """Same channels, kernel, groups and dtype on a smaller volume/shard plan."""
    spatial = tuple(int(s) for s in spatial)
    shards = tuple(tuple(int(v) for v in s) for s in shards)
    for ax, s in enumerate(shards):
        if sum(s) != spatial[ax]:
            raise ValueError("shard sizes must sum to the spatial extent")
    return dataclasses.replace(wl, name=f"{wl.name}_{name_suffix}", spatial=spatial,
                               shards=shards, batch=batch)
