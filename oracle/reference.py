"""Plain fp64 reference of what the halo-sharded layer computes.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Source.  "Technical summary: ShardTensor - domain parallelism for scientific
machine learning" (gist.science paper 2605.11111, Korean/Japanese/Spanish
versions of the same page):
  * section 2, "Design principles": with a batch of one, the spatial axes
    (height, width, depth) are split over devices, and every local chunk may
    have its own shape along the sharded axis ("sharding shapes");
  * section 2, "Implementation details", "Communication": collectives and a
    halo exchange (neighbouring pixels fetched from adjacent devices) keep
    convolution and normalisation numerically consistent with the unsharded
    computation.
The pages define neither convolution nor GroupNorm.  The readings taken here
(each is a textbook/PyTorch definition; ShardTensor extends PyTorch's DTensor,
section 2) are:
  * convolution = cross-correlation, stride 1, dilation 1, one group, odd
    cubic kernel, zero 'same' padding p = (k-1)/2, optional bias;
  * GroupNorm = contiguous channel groups, biased variance (divide by the
    element count M), eps inside the square root, per-channel affine;
  * halo width h = (k-1)/2 on every spatial axis; cells outside the global
    volume are zeros.
Arrays are channels-last: x is [N, *spatial, C] (the oracle only needs this to
be a fixed representation of the logical NC(D)HW tensor).

Nothing here is blocked, fused or reordered beyond the definitions: the conv
accumulates one tap at a time in lexicographic tap order, each tap a plain
matrix product over input channels.  The backward pass (training at native
resolution, section 1 "Problem statement" and the training runs of section
4) is the derivative of the same definitions: the input gradient, the weight
gradient and the GroupNorm backward, each pinned by tests/test_oracle.py.
"""
from __future__ import annotations

import itertools
from typing import Iterable, List, Sequence

import numpy as np


# ----------------------------------------------------------------------------
# representation helpers
# ----------------------------------------------------------------------------

def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of an fp32 array or of bf16 bit patterns (uint16)."""
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 operands are passed as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def zero_pad(x: np.ndarray, p: int) -> np.ndarray:
    """Zero-pad every spatial axis of a channels-last array by p on both sides."""
    d = x.ndim - 2
    return np.pad(x, [(0, 0)] + [(p, p)] * d + [(0, 0)])


# ----------------------------------------------------------------------------
# convolution (cross-correlation)
# ----------------------------------------------------------------------------

def _taps(k: int, d: int):
    """All kernel offsets t in {0..k-1}^d, lexicographic."""
    return list(itertools.product(range(k), repeat=d))


def conv_valid(xp: np.ndarray, w: np.ndarray, bias=None) -> np.ndarray:
    """Valid cross-correlation of an already padded volume.

    y[n, i, o] = b[o] + sum_t sum_c w[o, c, t] * xp[n, i + t, c]
    for every i with i + t inside xp.  xp: [N, *S_padded, Cin] fp64,
    w: [Cout, Cin, k, .., k] fp64.  Returns [N, *S_out, Cout] fp64.
    """
    d = xp.ndim - 2
    cout, cin = w.shape[:2]
    k = w.shape[2]
    if xp.shape[-1] != cin:
        raise ValueError("channel mismatch")
    s_out = [xp.shape[1 + a] - k + 1 for a in range(d)]
    y = np.zeros((xp.shape[0], *s_out, cout), dtype=np.float64)
    if bias is not None:
        y += np.asarray(bias, dtype=np.float64)
    for t in _taps(k, d):
        window = xp[(slice(None),) + tuple(slice(t[a], t[a] + s_out[a]) for a in range(d))]
        # [Cin, Cout] of this tap, contiguous so the product goes to BLAS
        wt = np.ascontiguousarray(w[(slice(None), slice(None)) + t].T)
        rows = np.ascontiguousarray(window).reshape(-1, cin)
        y += (rows @ wt).reshape(y.shape)
    return y


def conv_same(x: np.ndarray, w: np.ndarray, bias=None) -> np.ndarray:
    """'Same' cross-correlation with zero padding (k-1)/2 of an unpadded volume."""
    k = w.shape[2]
    if k % 2 != 1:
        raise ValueError("odd kernels only")
    return conv_valid(zero_pad(x, (k - 1) // 2), w, bias)


def conv_same_dgrad(dy: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Gradient of conv_same with respect to its input (its adjoint).

    The backward pass that training at native resolution needs ("Technical
    summary: ShardTensor", section 1 "Problem statement": training and
    inference on high-resolution data; section 4 "Results and benchmarks":
    ViT training at 2048^2, the StormScope training run):
    from y[n, i, o] = sum_t sum_c w[o, c, t] * x[n, i + t - p, c],
        dx[n, j, c] = sum_t sum_o w[o, c, t] * dy[n, j - t + p, o],
    with dy taken as zero outside the grid.  dy: [N, *S, Cout] fp64, w:
    [Cout, Cin, k, .., k] fp64; returns [N, *S, Cin] fp64.  One tap at a time,
    lexicographic, each a plain matrix product over output channels.
    """
    d = dy.ndim - 2
    cout, cin = w.shape[:2]
    k = w.shape[2]
    if k % 2 != 1:
        raise ValueError("odd kernels only")
    if dy.shape[-1] != cout:
        raise ValueError("channel mismatch")
    p = (k - 1) // 2
    S = dy.shape[1:1 + d]
    dyp = zero_pad(dy, p)                       # dyp[m] = dy[m - p]
    dx = np.zeros((dy.shape[0], *S, cin), dtype=np.float64)
    for t in _taps(k, d):
        # dy[j - t + p] = dyp[j - t + 2p]: the window starting at 2p - t
        window = dyp[(slice(None),) + tuple(slice(2 * p - t[a], 2 * p - t[a] + S[a]) for a in range(d))]
        rows = np.ascontiguousarray(window).reshape(-1, cout)
        wt = np.ascontiguousarray(w[(slice(None), slice(None)) + t])      # [Cout, Cin]
        dx += (rows @ wt).reshape(dx.shape)
    return dx


def conv_same_wgrad(x: np.ndarray, dy: np.ndarray, k: int) -> np.ndarray:
    """Gradient of conv_same with respect to its weights.

    The weight half of the backward pass (same passages as conv_same_dgrad).
    y[n, i, o] = sum_t sum_c w[o, c, t] * x[n, i + t - p, c] is linear in w, so
        dw[o, c, t] = sum_n sum_i dy[n, i, o] * x[n, i + t - p, c]
    with x taken as zero outside the grid.  x: [N, *S, Cin] fp64, dy:
    [N, *S, Cout] fp64; returns [Cout, Cin, k, .., k] fp64.  One tap at a
    time, lexicographic, each a plain matrix product over all positions.
    """
    d = x.ndim - 2
    if k % 2 != 1:
        raise ValueError("odd kernels only")
    if x.shape[:-1] != dy.shape[:-1]:
        raise ValueError("x and dy must share batch and spatial extents")
    cin, cout = x.shape[-1], dy.shape[-1]
    p = (k - 1) // 2
    S = x.shape[1:1 + d]
    xp = zero_pad(x, p)                          # xp[m] = x[m - p]
    g = np.ascontiguousarray(dy).reshape(-1, cout)
    dw = np.zeros((cout, cin) + (k,) * d, dtype=np.float64)
    for t in _taps(k, d):
        # x[i + t - p] = xp[i + t]: the window starting at t
        window = xp[(slice(None),) + tuple(slice(t[a], t[a] + S[a]) for a in range(d))]
        cols = np.ascontiguousarray(window).reshape(-1, cin)
        dw[(slice(None), slice(None)) + t] = g.T @ cols
    return dw


def conv_same_slabbed(x_src, dtype: str, w: np.ndarray, bias=None, slab: int = 8, start: int = 0,
                      stop=None):
    """conv_same evaluated one slab of the outermost spatial axis at a time.

    x_src is the (possibly bf16-bit) channels-last input; each output slab is
    the same definition restricted to those output positions, computed from
    the input rows it needs (zeros outside the volume).  Yields
    (start, y_slab) for the output rows [start, stop) of that axis (default:
    all of them).  This only bounds memory for the largest volumes.
    """
    k = w.shape[2]
    p = (k - 1) // 2
    n0 = x_src.shape[1]
    stop = n0 if stop is None else min(n0, stop)
    for s0 in range(start, stop, slab):
        s1 = min(stop, s0 + slab)
        lo, hi = s0 - p, s1 + p
        part = widen(x_src[:, max(0, lo):min(n0, hi)], dtype)
        pad_lo, pad_hi = max(0, -lo), max(0, hi - n0)
        part = np.pad(part, [(0, 0), (pad_lo, pad_hi)] + [(0, 0)] * (x_src.ndim - 2))
        # pad the remaining spatial axes fully
        d = x_src.ndim - 2
        part = np.pad(part, [(0, 0), (0, 0)] + [(p, p)] * (d - 1) + [(0, 0)])
        yield s0, conv_valid(part, w, bias)


def conv_at(x_src, dtype: str, w: np.ndarray, bias, positions: np.ndarray) -> np.ndarray:
    """y at selected output positions, each as one plain dot product.

    positions: [P, 1 + d] rows (n, i_0, .., i_{d-1}).  Input cells outside the
    volume count as zeros.  Returns [P, Cout] fp64.
    """
    d = x_src.ndim - 2
    k = w.shape[2]
    p = (k - 1) // 2
    cout, cin = w.shape[:2]
    wmat = w.reshape(cout, cin, -1)                       # [Cout, Cin, taps]
    out = np.zeros((len(positions), cout), dtype=np.float64)
    spatial = x_src.shape[1:-1]
    for r, pos in enumerate(positions):
        n = int(pos[0])
        centre = [int(v) for v in pos[1:]]
        window = np.zeros((k,) * d + (cin,), dtype=np.float64)
        src, dst = [n], []
        for a in range(d):
            lo = centre[a] - p
            a0, a1 = max(0, lo), min(spatial[a], lo + k)
            src.append(slice(a0, a1))
            dst.append(slice(a0 - lo, a1 - lo))
        window[tuple(dst)] = widen(x_src[tuple(src)], dtype)
        # window[t..., c] -> [Cin, taps] in the same tap order as w
        wc = np.moveaxis(window, -1, 0).reshape(cin, -1)
        out[r] = (wmat * wc[None]).sum(axis=(1, 2))
        if bias is not None:
            out[r] += np.asarray(bias, dtype=np.float64)
    return out


# ----------------------------------------------------------------------------
# GroupNorm
# ----------------------------------------------------------------------------

def _grouped(y: np.ndarray, groups: int) -> np.ndarray:
    n, c = y.shape[0], y.shape[-1]
    if c % groups:
        raise ValueError("channels must divide into groups")
    return y.reshape(n, -1, groups, c // groups)          # [N, positions, G, C/G]


def group_moments(y: np.ndarray, groups: int):
    """Two-pass mean and biased variance per (n, g): [N, G] each."""
    yg = _grouped(y, groups)
    mean = yg.mean(axis=(1, 3))
    var = ((yg - mean[:, None, :, None]) ** 2).mean(axis=(1, 3))
    return mean, var


def group_sums_onepass(y: np.ndarray, groups: int):
    """Element count M and the sums (sum y, sum y^2) per (n, g)."""
    yg = _grouped(y, groups)
    m = yg.shape[1] * yg.shape[3]
    return m, yg.sum(axis=(1, 3)), (yg * yg).sum(axis=(1, 3))


def group_norm_apply(y: np.ndarray, groups: int, mean, var, eps: float,
                     gamma=None, beta=None) -> np.ndarray:
    """z = (y - mean_g) / sqrt(var_g + eps) * gamma_c + beta_c."""
    c = y.shape[-1]
    gs = c // groups
    mean_c = np.repeat(np.asarray(mean, np.float64), gs, axis=-1)   # [N, C]
    var_c = np.repeat(np.asarray(var, np.float64), gs, axis=-1)
    shape = (y.shape[0],) + (1,) * (y.ndim - 2) + (c,)
    z = (y - mean_c.reshape(shape)) / np.sqrt(var_c.reshape(shape) + eps)
    if gamma is not None:
        z = z * np.asarray(gamma, np.float64)
    if beta is not None:
        z = z + np.asarray(beta, np.float64)
    return z


def group_norm(y: np.ndarray, groups: int, eps: float, gamma=None, beta=None) -> np.ndarray:
    mean, var = group_moments(y, groups)
    return group_norm_apply(y, groups, mean, var, eps, gamma, beta)


def group_norm_backward(y: np.ndarray, dz: np.ndarray, groups: int, eps: float, gamma=None):
    """Gradients of z = group_norm(y, groups, eps, gamma, beta) for an upstream
    gradient dz: (dy, dgamma, dbeta).

    The backward pass that training at native resolution needs ("Technical
    summary: ShardTensor", section 1 "Problem statement"; section 4 "Results
    and benchmarks", the training runs), for the GroupNorm read of the
    forward pass.  Per (n, g), with M elements, mean mu, biased variance var,
    r = 1 / sqrt(var + eps), yhat = (y - mu) * r and g = gamma_c * dz:
        dy     = r * (g - mean_g(g) - yhat * mean_g(g * yhat))
        dgamma = sum over n and positions of dz * yhat      (per channel)
        dbeta  = sum over n and positions of dz             (per channel)
    y, dz: [N, *S, C] fp64; returns dy [N, *S, C], dgamma [C], dbeta [C].
    """
    y = np.asarray(y, np.float64)
    dz = np.asarray(dz, np.float64)
    c = y.shape[-1]
    gamma = np.ones(c) if gamma is None else np.asarray(gamma, np.float64)
    mean, var = group_moments(y, groups)
    r = 1.0 / np.sqrt(var + eps)                                # [N, G]
    yg = _grouped(y, groups)                                    # [N, P, G, C/G]
    dzg = _grouped(dz, groups)
    yhat = (yg - mean[:, None, :, None]) * r[:, None, :, None]
    gg = dzg * gamma.reshape(groups, c // groups)
    m1 = gg.mean(axis=(1, 3))                                   # mean_g(g)
    m2 = (gg * yhat).mean(axis=(1, 3))                          # mean_g(g * yhat)
    dy = r[:, None, :, None] * (gg - m1[:, None, :, None] - yhat * m2[:, None, :, None])
    dgamma = (dzg * yhat).sum(axis=(0, 1)).reshape(c)
    dbeta = dzg.sum(axis=(0, 1)).reshape(c)
    return dy.reshape(y.shape), dgamma, dbeta


# ----------------------------------------------------------------------------
# shape-changing ops: 'valid' pooling and the sharding shapes it implies
# ----------------------------------------------------------------------------

def pool_valid(x: np.ndarray, k: int, s: int, mode: str = "avg") -> np.ndarray:
    """'Valid' pooling with a cubic window k and stride s on every spatial axis.

    The shape-changing case of the dynamic sharding shapes ("Technical
    summary: ShardTensor", section 2 "Design principles": every local chunk
    carries its own shape, and an op may change it).  Output j along an axis
    of extent n covers inputs [j*s, j*s + k), j = 0 .. (n - k) // s.
    mode "avg": mean of the k^d window; "max": its maximum.
    x: [N, *S, C] fp64; returns [N, *S', C].
    """
    d = x.ndim - 2
    S = x.shape[1:1 + d]
    if any(n < k for n in S):
        raise ValueError("window larger than the volume")
    out_S = tuple((n - k) // s + 1 for n in S)
    acc = None
    for t in _taps(k, d):
        window = x[(slice(None),) + tuple(slice(t[a], t[a] + s * (out_S[a] - 1) + 1, s) for a in range(d))]
        if acc is None:
            acc = np.array(window, dtype=np.float64)
        elif mode == "max":
            acc = np.maximum(acc, window)
        else:
            acc = acc + window
    return acc / float(k ** d) if mode == "avg" else acc


def conv_strided(x: np.ndarray, w: np.ndarray, s: int, bias=None) -> np.ndarray:
    """Strided cross-correlation with zero padding p = (k-1)/2: the
    shape-changing (downsampling) convolution.

    y[n, j, o] = b[o] + sum_t sum_c w[o, c, t] * x[n, j*s + t - p, c], for
    j = 0 .. (n_in + 2p - k) // s on every spatial axis (x zero outside the
    grid).  s = 1 is conv_same.  x: [N, *S, Cin]; w: [Cout, Cin, k, .., k].
    One tap at a time, lexicographic, each a plain matrix product over input
    channels.
    """
    d = x.ndim - 2
    cout, cin = w.shape[:2]
    k = w.shape[2]
    if k % 2 != 1:
        raise ValueError("odd kernels only")
    p = (k - 1) // 2
    S = x.shape[1:1 + d]
    out_S = tuple((n + 2 * p - k) // s + 1 for n in S)
    xp = zero_pad(x, p)
    y = np.zeros((x.shape[0], *out_S, cout), dtype=np.float64)
    if bias is not None:
        y += np.asarray(bias, np.float64)
    for t in _taps(k, d):
        window = xp[(slice(None),) + tuple(slice(t[a], t[a] + s * (out_S[a] - 1) + 1, s) for a in range(d))]
        rows = np.ascontiguousarray(window).reshape(-1, cin)
        wt = np.ascontiguousarray(w[(slice(None), slice(None)) + t]).T      # [Cin, Cout]
        y += (rows @ wt).reshape(y.shape)
    return y


def conv_transposed(y: np.ndarray, w: np.ndarray, s: int) -> np.ndarray:
    """Transposed (upsampling) convolution: the adjoint of conv_strided.

    With w [Cout, Cin, k, .., k] and p = (k-1)/2, every input cell i of y
    (Cout channels) adds sum_o w[o, c, t] * y[n, i, o] to output cell
    j = i*s + t - p (Cin channels) for every tap t; the output has s times the
    input's extent on every axis (cells j outside it are dropped).  So
    <conv_strided(x, w, s), y> = <x, conv_transposed(y, w, s)> for x of that
    extent.  One tap at a time, lexicographic, each a plain matrix product
    over the input channels.
    """
    d = y.ndim - 2
    cout, cin = w.shape[:2]
    k = w.shape[2]
    if k % 2 != 1:
        raise ValueError("odd kernels only")
    if y.shape[-1] != cout:
        raise ValueError("channel mismatch")
    p = (k - 1) // 2
    S = y.shape[1:1 + d]
    out_S = tuple(n * s for n in S)
    # scatter into an output padded by p on both sides, then crop
    big = np.zeros((y.shape[0], *[m + 2 * p + s for m in out_S], cin), dtype=np.float64)
    rows = np.ascontiguousarray(y).reshape(-1, cout)
    for t in _taps(k, d):
        wt = np.ascontiguousarray(w[(slice(None), slice(None)) + t])        # [Cout, Cin]
        contrib = (rows @ wt).reshape(y.shape[:-1] + (cin,))
        # j + p = i*s + t in the padded output
        idx = (slice(None),) + tuple(slice(t[a], t[a] + s * (S[a] - 1) + 1, s) for a in range(d))
        big[idx] += contrib
    crop = (slice(None),) + tuple(slice(p, p + out_S[a]) for a in range(d))
    return big[crop]


def strided_shard_sizes(sizes: Sequence[int], k: int, s: int) -> List[int]:
    """Output sharding shape of conv_strided along one axis: output j belongs
    to the shard whose interior holds its window's centre, input j*s."""
    n = int(sum(sizes))
    p = (k - 1) // 2
    n_out = (n + 2 * p - k) // s + 1
    out = []
    for a, e in zip(shard_offsets(sizes), sizes):
        first = -(-a // s)
        end = min(-(-(a + e) // s), n_out)
        out.append(end - first)
    return out


def pooled_shard_sizes(sizes: Sequence[int], k: int, s: int) -> List[int]:
    """Output sharding shape along one axis: output j belongs to the shard
    whose interior holds the first cell of its window, j*s."""
    n = int(sum(sizes))
    n_out = (n - k) // s + 1
    out = []
    for a, e in zip(shard_offsets(sizes), sizes):
        first = -(-a // s)                           # ceil(a / s)
        end = min(-(-(a + e) // s), n_out)
        out.append(end - first)
    return out


# ----------------------------------------------------------------------------
# sharding shapes and halos (the method's data movement, stated on arrays)
# ----------------------------------------------------------------------------

def shard_offsets(sizes: Sequence[int]) -> List[int]:
    """Start index of every shard along one axis (low index first)."""
    off = [0]
    for s in sizes:
        off.append(off[-1] + int(s))
    return off[:-1]


def shard_grid(shards: Sequence[Sequence[int]]):
    """All shard grid indices, row-major over the per-axis shard counts."""
    return list(itertools.product(*[range(len(s)) for s in shards]))


def padded_shard(x: np.ndarray, shards, index, h: int) -> np.ndarray:
    """What a shard's halo-padded buffer must hold after the exchange.

    It is the shard's box widened by h on every face, cut from the globally
    zero-padded volume: interior = the shard's cells, margins = neighbours'
    cells where a neighbour exists and zeros on the global faces.
    """
    xp = zero_pad(x, h)
    sl = [slice(None)]
    for a, sizes in enumerate(shards):
        o = shard_offsets(sizes)[index[a]]
        e = sizes[index[a]]
        sl.append(slice(o, o + e + 2 * h))               # padded coordinates
    return xp[tuple(sl)]


def halo_directions(d: int):
    """Neighbour directions delta in {-1,0,1}^d without 0, lexicographic."""
    return [t for t in itertools.product((-1, 0, 1), repeat=d) if any(t)]


def halo_message(x: np.ndarray, shards, h: int, align: int = 16) -> bytes:
    """The packed halo message: every box a shard sends to a neighbour.

    Order: source shard (row-major over the grid), then direction delta
    (lexicographic) towards the receiving neighbour, skipping directions with
    no neighbour.  The box sent in direction delta is, along each axis, the
    last h interior cells (delta=+1), the first h (delta=-1) or the whole
    interior extent (delta=0).  Each box is laid out channels-last in
    (n, *spatial, c) order and starts at a multiple of `align` bytes; bytes
    between boxes are zero.
    """
    d = x.ndim - 2
    out = bytearray()
    counts = [len(s) for s in shards]
    for idx in shard_grid(shards):
        for delta in halo_directions(d):
            nb = [idx[a] + delta[a] for a in range(d)]
            if any(nb[a] < 0 or nb[a] >= counts[a] for a in range(d)):
                continue
            sl = [slice(None)]
            for a in range(d):
                o = shard_offsets(shards[a])[idx[a]]
                e = shards[a][idx[a]]
                if delta[a] == 1:
                    sl.append(slice(o + e - h, o + e))
                elif delta[a] == -1:
                    sl.append(slice(o, o + h))
                else:
                    sl.append(slice(o, o + e))
            pad = (-len(out)) % align
            out += b"\0" * pad
            out += np.ascontiguousarray(x[tuple(sl)]).tobytes()
    return bytes(out)


def sharded_forward(x: np.ndarray, w: np.ndarray, bias, shards, groups: int,
                    eps: float, gamma=None, beta=None):
    """The method's steps on one host: halo-padded shards, per-shard conv,
    per-shard partial (count, sum, sum of squares), a combine over shards,
    then the apply.  Returns (y, z, per-shard partials) with y and z
    reassembled into the global [N, *spatial, Cout] arrays.
    """
    d = x.ndim - 2
    k = w.shape[2]
    h = (k - 1) // 2
    n = x.shape[0]
    cout = w.shape[0]
    y = np.zeros((n, *x.shape[1:-1], cout), dtype=np.float64)
    partials = []
    for idx in shard_grid(shards):
        chunk = padded_shard(x, shards, idx, h)
        ys = conv_valid(chunk, w, bias)
        partials.append(group_sums_onepass(ys, groups))
        sl = [slice(None)]
        for a in range(d):
            o = shard_offsets(shards[a])[idx[a]]
            sl.append(slice(o, o + shards[a][idx[a]]))
        y[tuple(sl)] = ys
    m = sum(p[0] for p in partials)
    s1 = sum(p[1] for p in partials)
    s2 = sum(p[2] for p in partials)
    mean = s1 / m
    var = s2 / m - mean * mean
    z = group_norm_apply(y, groups, mean, var, eps, gamma, beta)
    return y, z, partials


# ----------------------------------------------------------------------------
# brute force (scalar loops; tiny volumes only)
# ----------------------------------------------------------------------------

def conv_bruteforce(x, w, bias=None):
    """Scalar-loop 'same' cross-correlation with zero padding (tiny inputs)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    n_, *spatial, cin = x.shape
    d = len(spatial)
    cout, _, k = w.shape[:3]
    p = (k - 1) // 2
    y = np.zeros((n_, *spatial, cout))
    for n in range(n_):
        for pos in itertools.product(*[range(s) for s in spatial]):
            for o in range(cout):
                acc = 0.0 if bias is None else float(bias[o])
                for t in itertools.product(range(k), repeat=d):
                    src = [pos[a] + t[a] - p for a in range(d)]
                    if any(src[a] < 0 or src[a] >= spatial[a] for a in range(d)):
                        continue
                    for c in range(cin):
                        acc += w[(o, c) + t] * x[(n, *src, c)]
                y[(n, *pos, o)] = acc
    return y


def conv_dgrad_bruteforce(dy, w):
    """Scalar-loop input gradient of the 'same' cross-correlation (tiny inputs):
    every output position scatters w[o, c, t] * dy[o] onto the input position
    it read, exactly as the forward definition pairs them."""
    dy = np.asarray(dy, np.float64)
    w = np.asarray(w, np.float64)
    n_, *spatial, cout = dy.shape
    d = len(spatial)
    cin, k = w.shape[1], w.shape[2]
    p = (k - 1) // 2
    dx = np.zeros((n_, *spatial, cin))
    for n in range(n_):
        for pos in itertools.product(*[range(s) for s in spatial]):
            for t in itertools.product(range(k), repeat=d):
                src = [pos[a] + t[a] - p for a in range(d)]
                if any(src[a] < 0 or src[a] >= spatial[a] for a in range(d)):
                    continue
                for o in range(cout):
                    g = dy[(n, *pos, o)]
                    for c in range(cin):
                        dx[(n, *src, c)] += w[(o, c) + t] * g
    return dx


def conv_wgrad_bruteforce(x, dy, k):
    """Scalar-loop weight gradient of the 'same' cross-correlation (tiny
    inputs): every output position adds dy[o] * x[c] of the input cell that
    tap t of the forward definition reads."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    n_, *spatial, cin = x.shape
    cout = dy.shape[-1]
    d = len(spatial)
    p = (k - 1) // 2
    dw = np.zeros((cout, cin) + (k,) * d)
    for n in range(n_):
        for pos in itertools.product(*[range(s) for s in spatial]):
            for t in itertools.product(range(k), repeat=d):
                src = [pos[a] + t[a] - p for a in range(d)]
                if any(src[a] < 0 or src[a] >= spatial[a] for a in range(d)):
                    continue
                for o in range(cout):
                    for c in range(cin):
                        dw[(o, c) + t] += dy[(n, *pos, o)] * x[(n, *src, c)]
    return dw


def conv_strided_bruteforce(x, w, s, bias=None):
    """Scalar-loop strided 'same'-padded cross-correlation (tiny inputs)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    n_, *spatial, cin = x.shape
    d = len(spatial)
    cout, k = w.shape[0], w.shape[2]
    p = (k - 1) // 2
    out_S = [(m + 2 * p - k) // s + 1 for m in spatial]
    y = np.zeros((n_, *out_S, cout))
    for n in range(n_):
        for pos in itertools.product(*[range(m) for m in out_S]):
            for o in range(cout):
                acc = 0.0 if bias is None else float(bias[o])
                for t in itertools.product(range(k), repeat=d):
                    src = [pos[a] * s + t[a] - p for a in range(d)]
                    if any(src[a] < 0 or src[a] >= spatial[a] for a in range(d)):
                        continue
                    for c in range(cin):
                        acc += w[(o, c) + t] * x[(n, *src, c)]
                y[(n, *pos, o)] = acc
    return y


def conv_transposed_bruteforce(y, w, s):
    """Scalar-loop transposed convolution (tiny inputs): each input cell
    scatters w[o, c, t] * y[o] onto output cell i*s + t - p."""
    y = np.asarray(y, np.float64)
    w = np.asarray(w, np.float64)
    n_, *spatial, cout = y.shape
    d = len(spatial)
    cin, k = w.shape[1], w.shape[2]
    p = (k - 1) // 2
    out_S = [m * s for m in spatial]
    x = np.zeros((n_, *out_S, cin))
    for n in range(n_):
        for pos in itertools.product(*[range(m) for m in spatial]):
            for t in itertools.product(range(k), repeat=d):
                dst = [pos[a] * s + t[a] - p for a in range(d)]
                if any(dst[a] < 0 or dst[a] >= out_S[a] for a in range(d)):
                    continue
                for o in range(cout):
                    for c in range(cin):
                        x[(n, *dst, c)] += w[(o, c) + t] * y[(n, *pos, o)]
    return x


def pool_bruteforce(x, k, s, mode="avg"):
    """Scalar-loop 'valid' pooling (tiny inputs)."""
    x = np.asarray(x, np.float64)
    n_, *spatial, c = x.shape
    d = len(spatial)
    out_S = [(n - k) // s + 1 for n in spatial]
    y = np.zeros((n_, *out_S, c))
    for n in range(n_):
        for pos in itertools.product(*[range(m) for m in out_S]):
            for ch in range(c):
                vals = [x[(n, *[pos[a] * s + t[a] for a in range(d)], ch)]
                        for t in itertools.product(range(k), repeat=d)]
                y[(n, *pos, ch)] = max(vals) if mode == "max" else sum(vals) / len(vals)
    return y


def group_norm_bruteforce(y, groups, eps, gamma=None, beta=None):
    """Scalar-loop GroupNorm (tiny inputs)."""
    y = np.asarray(y, np.float64)
    n_, c = y.shape[0], y.shape[-1]
    gs = c // groups
    flat = y.reshape(n_, -1, c)
    z = np.zeros_like(flat)
    for n in range(n_):
        for g in range(groups):
            vals = [flat[n, i, ch] for i in range(flat.shape[1]) for ch in range(g * gs, (g + 1) * gs)]
            mean = sum(vals) / len(vals)
            var = sum((v - mean) ** 2 for v in vals) / len(vals)
            for i in range(flat.shape[1]):
                for ch in range(g * gs, (g + 1) * gs):
                    v = (flat[n, i, ch] - mean) / np.sqrt(var + eps)
                    if gamma is not None:
                        v *= float(gamma[ch])
                    if beta is not None:
                        v += float(beta[ch])
                    z[n, i, ch] = v
    return z.reshape(y.shape)
