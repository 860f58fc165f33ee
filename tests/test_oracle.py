"""Pins of the fp64 oracle against things other than itself (CPU only).

Each pin is a property the mathematics fixes: brute-force scalar loops, the
identity and shift kernels, linearity, an independent library (torch fp64 on
the CPU), GroupNorm closed forms, and the method's own invariant that the
sharded computation equals the unsharded one (ShardTensor summary, section 2,
"Implementation details", "Communication").  `test_pins_catch_mutants` plants
plausible mistakes in copies of the oracle and checks some pin fails.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synth


def rng(seed):
    return np.random.default_rng(seed)


def rand_case(seed, d, n=2, cin=3, cout=5, spatial=None, k=3):
    r = rng(seed)
    spatial = spatial or ((5, 6, 7) if d == 3 else (9, 11))
    x = r.standard_normal((n, *spatial, cin))
    w = r.uniform(-1, 1, size=(cout, cin) + (k,) * d)
    b = r.uniform(-1, 1, size=cout)
    return x, w, b


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------- pin helpers
# Each takes the functions under test so the mutation test can reuse them.

def pin_bruteforce(conv, gn):
    ok = True
    for d, k in [(2, 3), (2, 5), (3, 3), (3, 5)]:
        x, w, b = rand_case(10 + d * 10 + k, d, k=k, spatial=(4, 5, 6) if d == 3 else (7, 9))
        y = conv(x, w, b)
        ok &= rel(y, oracle.conv_bruteforce(x, w, b)) <= 1e-13
        g = 5 if y.shape[-1] % 5 == 0 else 1
        r = rng(d * k)
        gamma, beta = r.uniform(0.5, 1.5, y.shape[-1]), r.uniform(-1, 1, y.shape[-1])
        ok &= rel(gn(y, g, 1e-5, gamma, beta),
                  oracle.group_norm_bruteforce(y, g, 1e-5, gamma, beta)) <= 1e-12
        # two groups of unequal content, to pin the channel-to-group map
        y2 = np.concatenate([y, 3.0 * y[..., :1] + 1.0], axis=-1)  # 6 channels
        ok &= rel(gn(y2, 2, 1e-5), oracle.group_norm_bruteforce(y2, 2, 1e-5)) <= 1e-12
    return bool(ok)


def pin_identity(conv):
    ok = True
    for d, k in [(2, 3), (3, 3), (3, 5)]:
        x, _, _ = rand_case(7, d, cin=4, cout=4, k=k)
        w = np.zeros((4, 4) + (k,) * d)
        c = (k // 2,) * d
        for o in range(4):
            w[(o, o) + c] = 1.0
        ok &= np.array_equal(conv(x, w, None), x)
    return bool(ok)


def pin_shift(conv):
    """A one-hot kernel at tap t moves x by t - p, with zeros entering at faces."""
    ok = True
    for d, k in [(2, 3), (3, 5)]:
        x, _, _ = rand_case(8, d, cin=2, cout=2, k=k)
        p = k // 2
        spatial = x.shape[1:-1]
        for t in [(0,) * d, (k - 1,) * d, tuple(range(d)), (k - 1,) + (0,) * (d - 1)]:
            w = np.zeros((2, 2) + (k,) * d)
            w[(0, 1) + t] = 1.0          # output 0 <- input channel 1
            w[(1, 0) + t] = 2.0          # output 1 <- 2 * input channel 0
            want = np.zeros(x.shape[:-1] + (2,))
            for pos in itertools.product(*[range(s) for s in spatial]):
                src = tuple(pos[a] + t[a] - p for a in range(d))
                if all(0 <= src[a] < spatial[a] for a in range(d)):
                    want[(slice(None),) + pos + (0,)] = x[(slice(None),) + src + (1,)]
                    want[(slice(None),) + pos + (1,)] = 2.0 * x[(slice(None),) + src + (0,)]
            ok &= np.array_equal(conv(x, w, None), want)
    return bool(ok)


def pin_linearity(conv):
    ok = True
    for d in (2, 3):
        x1, w1, _ = rand_case(21, d)
        x2, w2, _ = rand_case(22, d)
        a, c = 0.75, -1.5
        y = conv(a * x1 + c * x2, w1, None)
        ok &= rel(y, a * conv(x1, w1, None) + c * conv(x2, w1, None)) <= 1e-13
        y = conv(x1, a * w1 + c * w2, None)
        ok &= rel(y, a * conv(x1, w1, None) + c * conv(x1, w2, None)) <= 1e-13
    return bool(ok)


def pin_torch(conv, gn):
    """torch.nn.functional on the CPU in float64: an independent implementation."""
    ok = True
    for d, k in [(2, 3), (3, 3), (3, 5), (2, 5)]:
        x, w, b = rand_case(30 + d + k, d, n=2, cin=6, cout=8, k=k,
                            spatial=(6, 7, 9) if d == 3 else (12, 10))
        xt = torch.from_numpy(np.moveaxis(x, -1, 1).copy())
        f = torch.nn.functional.conv3d if d == 3 else torch.nn.functional.conv2d
        yt = f(xt, torch.from_numpy(w), torch.from_numpy(b), padding=k // 2)
        y = conv(x, w, b)
        ok &= rel(y, np.moveaxis(yt.numpy(), 1, -1)) <= 1e-12
        r = rng(d * 100 + k)
        gamma, beta = r.uniform(0.5, 1.5, 8), r.uniform(-1, 1, 8)
        zt = torch.nn.functional.group_norm(yt, 4, torch.from_numpy(gamma),
                                            torch.from_numpy(beta), eps=1e-5)
        ok &= rel(gn(y, 4, 1e-5, gamma, beta), np.moveaxis(zt.numpy(), 1, -1)) <= 1e-12
    return bool(ok)


def pin_groupnorm_closed_forms(gn):
    ok = True
    r = rng(5)
    y = r.standard_normal((2, 6, 7, 8)) * r.uniform(0.1, 3, 8) + r.uniform(-2, 2, 8)
    eps = 1e-5
    z = gn(y, 4, eps)
    zg = z.reshape(2, -1, 4, 2)
    yg = y.reshape(2, -1, 4, 2)
    var = yg.var(axis=(1, 3))
    ok &= np.max(np.abs(zg.mean(axis=(1, 3)))) < 1e-13
    ok &= rel(zg.var(axis=(1, 3)), var / (var + eps)) < 1e-12
    # constant groups normalise to beta
    beta = np.arange(8.0)
    zc = gn(np.full((1, 5, 5, 8), 3.25), 4, eps, None, beta)
    ok &= np.array_equal(zc, np.broadcast_to(beta, zc.shape))
    # eps = 0: z(a*y + c) = sign(a) * z(y)
    for a, c in [(2.5, 1.0), (-0.5, 3.0)]:
        ok &= rel(gn(a * y + c, 4, 0.0), np.sign(a) * gn(y, 4, 0.0)) < 1e-12
    return bool(ok)


def pin_sharded(conv, gn):
    """Sharded-with-halo conv + split-stat GroupNorm == unsharded (fp64)."""
    ok = True
    cases = [
        (2, 3, ((4, 3, 5), (12,))),
        (2, 3, ((12,), (5, 7))),
        (3, 3, ((3, 4), (2, 3, 3), (5, 4))),
        (3, 5, ((4, 2, 3), (9,), (4, 6))),
    ]
    for d, k, shards in cases:
        spatial = tuple(sum(s) for s in shards)
        x, w, b = rand_case(40 + d + k, d, n=2, cin=3, cout=4, k=k, spatial=spatial)
        y, z, partials = oracle.sharded_forward(x, w, b, shards, 2, 1e-5)
        ok &= rel(y, conv(x, w, b)) <= 1e-13
        ok &= rel(z, gn(conv(x, w, b), 2, 1e-5)) <= 1e-10
        ok &= len(partials) == int(np.prod([len(s) for s in shards]))
    return bool(ok)


def pin_dgrad(dgrad, conv=oracle.conv_same):
    """The input gradient against what fixes it independently: the adjoint
    identity <conv(x), dy> = <x, dgrad(dy)> (every x and dy), scalar-loop
    brute force on tiny volumes, and torch's fp64 autograd."""
    ok = True
    for d, k in [(2, 3), (2, 5), (3, 3), (3, 5)]:
        r = rng(500 + 10 * d + k)
        spatial = (5, 6, 7) if d == 3 else (9, 11)
        x = r.standard_normal((2, *spatial, 3))
        dy = r.standard_normal((2, *spatial, 4))
        w = r.uniform(-1, 1, size=(4, 3) + (k,) * d)
        y = conv(x, w)
        lhs = float(np.sum(y * dy))
        rhs = float(np.sum(x * dgrad(dy, w)))
        ok &= abs(lhs - rhs) <= 1e-13 * float(np.sum(np.abs(y * dy)))   # rounding of the two sums only
        small = (3, 4, 4) if d == 3 else (5, 6)
        dys = r.standard_normal((1, *small, 4))
        ok &= rel(dgrad(dys, w), oracle.conv_dgrad_bruteforce(dys, w)) <= 1e-13
        xt = torch.from_numpy(np.moveaxis(x, -1, 1).copy()).requires_grad_(True)
        f = torch.nn.functional.conv3d if d == 3 else torch.nn.functional.conv2d
        yt = f(xt, torch.from_numpy(w), padding=k // 2)
        yt.backward(torch.from_numpy(np.moveaxis(dy, -1, 1).copy()))
        ok &= rel(dgrad(dy, w), np.moveaxis(xt.grad.numpy(), 1, -1)) <= 1e-12
    return bool(ok)


def pin_wgrad(wgrad, conv=oracle.conv_same):
    """The weight gradient against what fixes it independently: the adjoint
    identity in the weights <conv(x, w), dy> = <w, wgrad(x, dy)> (conv is
    linear in w), scalar-loop brute force on tiny volumes, and torch's fp64
    autograd with respect to the weight."""
    ok = True
    for d, k in [(2, 3), (2, 5), (3, 3), (3, 5)]:
        r = rng(600 + 10 * d + k)
        spatial = (5, 6, 7) if d == 3 else (9, 11)
        x = r.standard_normal((2, *spatial, 3))
        dy = r.standard_normal((2, *spatial, 4))
        w = r.uniform(-1, 1, size=(4, 3) + (k,) * d)
        y = conv(x, w)
        lhs = float(np.sum(y * dy))
        rhs = float(np.sum(w * wgrad(x, dy, k)))
        ok &= abs(lhs - rhs) <= 1e-13 * float(np.sum(np.abs(y * dy)))
        small = (3, 4, 4) if d == 3 else (5, 6)
        xs, dys = r.standard_normal((2, *small, 3)), r.standard_normal((2, *small, 4))
        ok &= rel(wgrad(xs, dys, k), oracle.conv_wgrad_bruteforce(xs, dys, k)) <= 1e-13
        wt = torch.from_numpy(w.copy()).requires_grad_(True)
        f = torch.nn.functional.conv3d if d == 3 else torch.nn.functional.conv2d
        yt = f(torch.from_numpy(np.moveaxis(x, -1, 1).copy()), wt, padding=k // 2)
        yt.backward(torch.from_numpy(np.moveaxis(dy, -1, 1).copy()))
        ok &= rel(wgrad(x, dy, k), wt.grad.numpy()) <= 1e-12
    return bool(ok)


def pin_gn_backward(gnb, gn=oracle.group_norm):
    """GroupNorm backward against torch's fp64 autograd and central finite
    differences of the loss <group_norm(y), dz> (independent of the formula)."""
    ok = True
    for shape, groups in [((2, 5, 6, 8), 4), ((1, 3, 4, 5, 6), 2), ((2, 7, 4), 1)]:
        r = rng(700 + len(shape) + groups)
        y = r.standard_normal(shape) * 1.5 + 0.3
        dz = r.standard_normal(shape)
        c = shape[-1]
        gamma, beta = r.uniform(0.5, 1.5, c), r.uniform(-1, 1, c)
        dy, dg, db = gnb(y, dz, groups, 1e-5, gamma)
        yt = torch.from_numpy(np.moveaxis(y, -1, 1).copy()).requires_grad_(True)
        gt = torch.from_numpy(gamma.copy()).requires_grad_(True)
        bt = torch.from_numpy(beta.copy()).requires_grad_(True)
        zt = torch.nn.functional.group_norm(yt, groups, gt, bt, eps=1e-5)
        zt.backward(torch.from_numpy(np.moveaxis(dz, -1, 1).copy()))
        ok &= rel(dy, np.moveaxis(yt.grad.numpy(), 1, -1)) <= 1e-11
        ok &= rel(dg, gt.grad.numpy()) <= 1e-11 and rel(db, bt.grad.numpy()) <= 1e-11
        # finite differences of L(y) = <gn(y), dz> at a few coordinates
        for k in range(4):
            idx = tuple(int(r.integers(0, s_)) for s_ in shape)
            h = 1e-5
            yp, ym = y.copy(), y.copy()
            yp[idx] += h
            ym[idx] -= h
            fd = (np.sum(gn(yp, groups, 1e-5, gamma, beta) * dz) - np.sum(gn(ym, groups, 1e-5, gamma, beta) * dz)) / (2 * h)
            ok &= abs(fd - dy[idx]) <= 1e-6 * max(1.0, abs(dy[idx]))
    return bool(ok)


# ------------------------------------------------------------------- the pins

def test_gn_backward_pins():
    assert pin_gn_backward(oracle.group_norm_backward)


@pytest.mark.parametrize("name", ["mean term dropped", "yhat term dropped", "gamma ignored", "unbiased variance"])
def test_gn_backward_pins_catch_mutants(name):
    def no_mean(y, dz, g, eps, gamma=None):
        dy, dg, db = oracle.group_norm_backward(y, dz, g, eps, gamma)
        yg = dz.reshape(dz.shape[0], -1, g, dz.shape[-1] // g) * (1 if gamma is None else gamma).reshape(g, -1)
        m1 = yg.mean(axis=(1, 3))
        mean, var = oracle.group_moments(y, g)
        r = 1.0 / np.sqrt(var + eps)
        add = np.repeat(r * m1, dz.shape[-1] // g, axis=-1).reshape((dz.shape[0],) + (1,) * (dz.ndim - 2) + (-1,))
        return dy + add, dg, db

    def no_yhat(y, dz, g, eps, gamma=None):
        mean, var = oracle.group_moments(y, g)
        r = 1.0 / np.sqrt(var + eps)
        c = dz.shape[-1]
        gm = dz * (1 if gamma is None else gamma)
        gg = gm.reshape(dz.shape[0], -1, g, c // g)
        dy = r[:, None, :, None] * (gg - gg.mean(axis=(1, 3))[:, None, :, None])
        _, dg, db = oracle.group_norm_backward(y, dz, g, eps, gamma)
        return dy.reshape(dz.shape), dg, db

    def no_gamma(y, dz, g, eps, gamma=None):
        return oracle.group_norm_backward(y, dz, g, eps, None)

    def unbiased(y, dz, g, eps, gamma=None):
        m = y.size // (y.shape[0] * g)
        return oracle.group_norm_backward(y * np.sqrt(m / (m - 1)), dz, g, eps, gamma)

    mutant = {"mean term dropped": no_mean, "yhat term dropped": no_yhat, "gamma ignored": no_gamma,
              "unbiased variance": unbiased}[name]
    assert not pin_gn_backward(mutant), f"no pin caught the GroupNorm-backward mutant '{name}'"

def test_wgrad_pins():
    assert pin_wgrad(oracle.conv_same_wgrad)


@pytest.mark.parametrize("name", ["flipped taps", "channels swapped", "shift off by one", "batch not summed"])
def test_wgrad_pins_catch_mutants(name):
    def flipped(x, dy, k):
        dw = oracle.conv_same_wgrad(x, dy, k)
        return np.flip(dw, axis=tuple(range(2, dw.ndim))).copy()

    def swapped(x, dy, k):
        dw = oracle.conv_same_wgrad(x, dy, k)
        r = np.moveaxis(dw.reshape(dw.shape[0] * dw.shape[1], -1), 0, 0)
        return r[::-1].reshape(dw.shape)      # o and c indices scrambled

    def shifted(x, dy, k):
        return oracle.conv_same_wgrad(np.roll(x, 1, axis=1), dy, k)

    def one_sample(x, dy, k):
        return oracle.conv_same_wgrad(x[:1], dy[:1], k)

    mutant = {"flipped taps": flipped, "channels swapped": swapped, "shift off by one": shifted,
              "batch not summed": one_sample}[name]
    assert not pin_wgrad(mutant), f"no pin caught the wgrad mutant '{name}'"


def pin_pool(pool, sizes_fn=oracle.pooled_shard_sizes):
    """'Valid' pooling against scalar brute force, torch's fp64 pooling, and
    the method's own invariant: each shard pooled from its halo-padded chunk
    (outputs owned by the shard holding their window's first cell) equals
    the matching slice of the unsharded result.  A shape error counts as a
    failed pin."""
    try:
        return _pin_pool(pool, sizes_fn)
    except (ValueError, IndexError):
        return False


def _pin_pool(pool, sizes_fn):
    ok = True
    for d, k, s in [(2, 2, 2), (2, 3, 2), (3, 2, 2), (3, 3, 1), (2, 3, 3)]:
        r = rng(800 + 100 * d + 10 * k + s)
        spatial = (10, 9, 8) if d == 3 else (12, 13)
        x = r.standard_normal((2, *spatial, 3))
        for mode in ("avg", "max"):
            y = pool(x, k, s, mode)
            small = (4, 5, 5) if d == 3 else (6, 7)
            xs = r.standard_normal((1, *small, 2))
            ok &= rel(pool(xs, k, s, mode), oracle.pool_bruteforce(xs, k, s, mode)) <= 1e-13
            xt = torch.from_numpy(np.moveaxis(x, -1, 1).copy())
            if mode == "avg":
                f = torch.nn.functional.avg_pool3d if d == 3 else torch.nn.functional.avg_pool2d
            else:
                f = torch.nn.functional.max_pool3d if d == 3 else torch.nn.functional.max_pool2d
            ok &= rel(y, np.moveaxis(f(xt, k, s).numpy(), 1, -1)) <= 1e-13
        # sharded form along axis 0 with uneven sizes (odd boundaries straddle windows)
        sizes = [4, 3, spatial[0] - 7]
        out_sizes = sizes_fn(sizes, k, s)
        ok &= sum(out_sizes) == y.shape[1]
        h = k - 1
        xp = zero_pad_axis0(x, h)
        o0 = 0
        for a, e, m in zip(oracle.shard_offsets(sizes), sizes, out_sizes):
            padded = xp[:, a: a + e + 2 * h]           # the shard's chunk with its halo along axis 0
            first = -(-a // s)
            lo = first * s - a + h                      # first owned window, in padded coordinates
            if m == 0:                                  # a shard may own no window start
                continue
            ok &= lo + (m - 1) * s + k <= padded.shape[1]
            chunk = padded[:, lo: lo + (m - 1) * s + k]
            ok &= np.array_equal(pool(chunk, k, s, "max"), pool(x, k, s, "max")[:, o0:o0 + m])
            o0 += m
    return bool(ok)


def zero_pad_axis0(x, h):
    pad = [(0, 0)] * x.ndim
    pad[1] = (h, h)
    return np.pad(x, pad)


def test_pool_pins():
    assert pin_pool(oracle.pool_valid)


@pytest.mark.parametrize("name", ["window off by one", "stride ignored", "sum not mean", "last shard owns"])
def test_pool_pins_catch_mutants(name):
    def window(x, k, s, mode="avg"):
        return oracle.pool_valid(x, k + 1, s, mode) if min(x.shape[1:-1]) > k else oracle.pool_valid(x, k, s, mode) + 1

    def stride1(x, k, s, mode="avg"):
        return oracle.pool_valid(x, k, 1, mode)

    def summed(x, k, s, mode="avg"):
        y = oracle.pool_valid(x, k, s, mode)
        return y * (k ** (x.ndim - 2)) if mode == "avg" else y

    def last_owns(sizes, k, s):
        out = oracle.pooled_shard_sizes(sizes, k, s)
        return [o + (1 if i == len(out) - 1 else 0) for i, o in enumerate(out)]

    if name == "last shard owns":
        assert not pin_pool(oracle.pool_valid, last_owns)
        return
    mutant = {"window off by one": window, "stride ignored": stride1, "sum not mean": summed}[name]
    assert not pin_pool(mutant), f"no pin caught the pooling mutant '{name}'"


def pin_strided(conv, sizes_fn=oracle.strided_shard_sizes):
    """The strided conv against scalar brute force, torch's fp64 conv with
    stride and padding, the stride-1 case (conv_same), and the sharded form:
    each shard's owned outputs (window centre in its interior) computed from
    its halo-padded chunk equal the matching slice of the unsharded result."""
    try:
        ok = True
        for d, k, s in [(2, 3, 2), (2, 5, 2), (3, 3, 2), (2, 3, 3), (3, 3, 1)]:
            r = rng(900 + 100 * d + 10 * k + s)
            spatial = (10, 9, 8) if d == 3 else (12, 13)
            x = r.standard_normal((2, *spatial, 3))
            w = r.uniform(-1, 1, size=(4, 3) + (k,) * d)
            b = r.uniform(-1, 1, size=4)
            y = conv(x, w, s, b)
            small = (4, 5, 5) if d == 3 else (6, 7)
            xs = r.standard_normal((1, *small, 3))
            ok &= rel(conv(xs, w, s, b), oracle.conv_strided_bruteforce(xs, w, s, b)) <= 1e-13
            f = torch.nn.functional.conv3d if d == 3 else torch.nn.functional.conv2d
            yt = f(torch.from_numpy(np.moveaxis(x, -1, 1).copy()), torch.from_numpy(w), torch.from_numpy(b),
                   stride=s, padding=k // 2)
            ok &= rel(y, np.moveaxis(yt.numpy(), 1, -1)) <= 1e-12
            if s == 1:
                ok &= rel(y, oracle.conv_same(x, w, b)) <= 1e-13
            sizes = [4, 3, spatial[0] - 7]
            out_sizes = sizes_fn(sizes, k, s)
            ok &= sum(out_sizes) == y.shape[1]
            h = k // 2
            xp = zero_pad_axis0(x, h)
            o0 = 0
            for a, e, m in zip(oracle.shard_offsets(sizes), sizes, out_sizes):
                if m == 0:
                    continue
                padded = xp[:, a: a + e + 2 * h]         # the shard's chunk with its halo along axis 0
                first = -(-a // s)
                lo = first * s - a                        # first owned window, in padded coordinates
                ok &= lo + (m - 1) * s + k <= padded.shape[1]
                chunk = padded[:, lo: lo + (m - 1) * s + k]
                # torch: no padding along axis 0 (the halo is in the chunk), 'same' padding elsewhere
                pad = (0,) + (h,) * (d - 1)
                part = f(torch.from_numpy(np.moveaxis(chunk, -1, 1).copy()), torch.from_numpy(w),
                         torch.from_numpy(b), stride=s, padding=pad)
                ok &= rel(np.moveaxis(part.numpy(), 1, -1), y[:, o0:o0 + m]) <= 1e-12
                o0 += m
        return bool(ok)
    except (ValueError, IndexError, RuntimeError):
        return False


def pin_transposed(convt, conv=oracle.conv_strided):
    """The transposed conv against the adjoint identity with the strided conv
    <conv_strided(x, w, s), y> = <x, conv_transposed(y, w, s)>, scalar-loop
    brute force, torch's fp64 conv_transpose (padding k/2, output padding
    s - 1) and the sharded form: a shard's outputs [a*s, (a+e)*s) computed
    from its halo-padded input chunk equal the slice of the whole result."""
    try:
        ok = True
        for d, k, s in [(2, 3, 2), (2, 5, 2), (3, 3, 2), (2, 3, 3), (3, 3, 1)]:
            r = rng(950 + 100 * d + 10 * k + s)
            spatial = (5, 4, 6) if d == 3 else (7, 6)
            y = r.standard_normal((2, *spatial, 4))
            w = r.uniform(-1, 1, size=(4, 3) + (k,) * d)
            xt = convt(y, w, s)
            x = r.standard_normal(xt.shape)
            lhs = float(np.sum(conv(x, w, s) * y))
            rhs = float(np.sum(x * xt))
            ok &= abs(lhs - rhs) <= 1e-12 * float(np.sum(np.abs(conv(x, w, s) * y)))
            ys = r.standard_normal((1, *[max(2, m - 3) for m in spatial], 4))
            ok &= rel(convt(ys, w, s), oracle.conv_transposed_bruteforce(ys, w, s)) <= 1e-13
            f = torch.nn.functional.conv_transpose3d if d == 3 else torch.nn.functional.conv_transpose2d
            tt = f(torch.from_numpy(np.moveaxis(y, -1, 1).copy()), torch.from_numpy(w), stride=s, padding=k // 2,
                   output_padding=s - 1)
            ok &= rel(xt, np.moveaxis(tt.numpy(), 1, -1)) <= 1e-12
            # sharded along axis 0: shard [a, a+e) of y owns outputs [a*s, (a+e)*s)
            sizes = [2, 3, spatial[0] - 5]
            h = k // 2
            yp = zero_pad_axis0(y, h)
            for a, e in zip(oracle.shard_offsets(sizes), sizes):
                if e == 0:
                    continue
                chunk = yp[:, a: a + e + 2 * h]          # the shard's input with its halo along axis 0
                part = convt(chunk, w, s)[:, h * s: h * s + e * s]
                ok &= rel(part, xt[:, a * s: (a + e) * s]) <= 1e-12
        return bool(ok)
    except (ValueError, IndexError, RuntimeError):
        return False


def test_transposed_pins():
    assert pin_transposed(oracle.conv_transposed)


@pytest.mark.parametrize("name", ["taps not flipped", "stride ignored", "no crop offset"])
def test_transposed_pins_catch_mutants(name):
    def unflipped(y, w, s):
        return oracle.conv_transposed(y, np.flip(w, axis=tuple(range(2, w.ndim))).copy(), s)

    def stride1(y, w, s):
        out = oracle.conv_transposed(y, w, 1)
        reps = [1] + [s] * (y.ndim - 2) + [1]
        return np.kron(out, np.ones(reps)) if s > 1 else out

    def shifted(y, w, s):
        return np.roll(oracle.conv_transposed(y, w, s), 1, axis=1)

    mutant = {"taps not flipped": unflipped, "stride ignored": stride1, "no crop offset": shifted}[name]
    assert not pin_transposed(mutant), f"no pin caught the transposed-conv mutant '{name}'"


def test_strided_pins():
    assert pin_strided(oracle.conv_strided)


@pytest.mark.parametrize("name", ["stride ignored", "no padding offset", "owner by window start"])
def test_strided_pins_catch_mutants(name):
    def stride1(x, w, s, b=None):
        return oracle.conv_strided(x, w, 1, b)

    def nopad(x, w, s, b=None):
        y = oracle.conv_strided(x, w, s, b)
        return np.roll(y, 1, axis=1)

    def start_owner(sizes, k, s):
        return oracle.pooled_shard_sizes(sizes, k, s)

    if name == "owner by window start":
        assert not pin_strided(oracle.conv_strided, start_owner)
        return
    mutant = {"stride ignored": stride1, "no padding offset": nopad}[name]
    assert not pin_strided(mutant), f"no pin caught the strided-conv mutant '{name}'"


def test_dgrad_pins():
    assert pin_dgrad(oracle.conv_same_dgrad)


@pytest.mark.parametrize("name", ["unflipped taps", "untransposed channels", "shift off by one"])
def test_dgrad_pins_catch_mutants(name):
    def unflipped(dy, w):
        return oracle.conv_same(dy, np.swapaxes(w, 0, 1).copy())

    def untransposed(dy, w):
        if w.shape[0] == w.shape[1]:
            return oracle.conv_same(dy, np.flip(w, axis=tuple(range(2, w.ndim))).copy())
        return oracle.conv_same_dgrad(dy, w) * (1 + 1e-9)

    def shifted(dy, w):
        return np.roll(oracle.conv_same_dgrad(dy, w), 1, axis=1)

    mutant = {"unflipped taps": unflipped, "untransposed channels": untransposed,
              "shift off by one": shifted}[name]
    assert not pin_dgrad(mutant), f"no pin caught the dgrad mutant '{name}'"

def test_bruteforce():
    assert pin_bruteforce(oracle.conv_same, oracle.group_norm)


def test_identity_kernel_exact():
    assert pin_identity(oracle.conv_same)


def test_shift_kernel_exact():
    assert pin_shift(oracle.conv_same)


def test_linearity():
    assert pin_linearity(oracle.conv_same)


def test_torch_fp64():
    assert pin_torch(oracle.conv_same, oracle.group_norm)


def test_groupnorm_closed_forms():
    assert pin_groupnorm_closed_forms(oracle.group_norm)


def test_sharded_equals_unsharded():
    assert pin_sharded(oracle.conv_same, oracle.group_norm)


def test_onepass_sums_agree_with_two_pass():
    r = rng(3)
    y = r.standard_normal((1, 9, 10, 8)) * 2 + 0.5
    m, s1, s2 = oracle.group_sums_onepass(y, 4)
    mean, var = oracle.group_moments(y, 4)
    assert m == 9 * 10 * 2
    assert rel(s1 / m, mean) < 1e-13
    assert np.max(np.abs((s2 / m - (s1 / m) ** 2) - var)) <= 1e-10 * np.max(var)


def test_conv_box_sum_closed_form():
    """All-ones 3x3 kernel on a ramp: each output is the sum of the in-bounds
    3x3 neighbourhood, which for x[i, j] = i + 10 j has a closed form."""
    H, W = 5, 6
    i, j = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
    x = (i + 10.0 * j)[None, :, :, None]
    w = np.ones((1, 1, 3, 3))
    y = oracle.conv_same(x, w)[0, :, :, 0]
    for a in range(H):
        for b in range(W):
            rows = [r for r in (a - 1, a, a + 1) if 0 <= r < H]
            cols = [c for c in (b - 1, b, b + 1) if 0 <= c < W]
            want = len(cols) * sum(rows) + 10.0 * len(rows) * sum(cols)
            assert y[a, b] == want


def test_conv_at_matches_full_conv():
    wl = synth.small_variant(synth.workload("vol512_c16_k5_bf16"), (12, 9, 10),
                             ((5, 7), (9,), (10,)))
    x = synth.make_input(wl)
    w = oracle.widen(synth.make_weight(wl), "bf16")
    y = oracle.conv_same(oracle.widen(x, "bf16"), w)
    pos = synth.sample_positions(wl, 64, 1)
    got = oracle.conv_at(x, "bf16", w, None, pos)
    want = np.stack([y[tuple(p)] for p in pos])
    assert rel(got, want) < 1e-13


def test_slabbed_conv_matches_full_conv():
    for name in ["vol512_c16_k5_bf16", "img2048_c64_k3_bf16"]:
        base = synth.workload(name)
        sp = (11, 9, 8)[:base.ndim]
        wl = synth.small_variant(base, sp, [(s,) for s in sp])
        x = synth.make_input(wl)
        w = oracle.widen(synth.make_weight(wl), "bf16")
        y = oracle.conv_same(oracle.widen(x, "bf16"), w)
        parts = [ys for _, ys in oracle.conv_same_slabbed(x, "bf16", w, None, slab=3)]
        assert np.array_equal(np.concatenate(parts, axis=1), y)
        # a row range: exactly those rows of the full conv, boundary rows included
        for lo, hi in [(0, 2), (4, 9), (9, 11), (10, 30)]:
            got = [(s0, ys) for s0, ys in oracle.conv_same_slabbed(x, "bf16", w, None, slab=2, start=lo, stop=hi)]
            assert got[0][0] == lo
            assert np.array_equal(np.concatenate([ys for _, ys in got], axis=1), y[:, lo:min(hi, sp[0])])


# ------------------------------------------------------------ halo reference

def test_padded_shard_is_neighbourhood_with_zero_faces():
    r = rng(9)
    x = r.standard_normal((1, 7, 8, 2))
    shards = ((3, 4), (5, 3))
    h = 1
    got = oracle.padded_shard(x, shards, (1, 0), h)
    # shard (1, 0) covers rows 3..6, cols 0..4; padded rows 2..7, cols -1..5
    want = np.zeros((1, 6, 7, 2))
    for a in range(6):
        for b in range(7):
            r_, c_ = 2 + a, -1 + b
            if 0 <= r_ < 7 and 0 <= c_ < 8:
                want[0, a, b] = x[0, r_, c_]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("shards,h", [
    (((3, 4), (5, 3)), 1),
    (((4, 3, 5), (6,)), 2),
    (((3, 4), (2, 3), (4, 3)), 1),
    (((5, 4, 6), (7,), (6,)), 2),
])
def test_halo_message_fills_every_margin(shards, h):
    """Placing every message box into the receiver's margin, plus zeros on the
    global faces, must rebuild each padded shard exactly."""
    d = len(shards)
    spatial = tuple(sum(s) for s in shards)
    x = rng(11).standard_normal((2, *spatial, 3))
    msg = np.frombuffer(oracle.halo_message(x, shards, h), dtype=np.float64)
    counts = [len(s) for s in shards]
    bufs = {}
    for idx in oracle.shard_grid(shards):
        ext = [shards[a][idx[a]] for a in range(d)]
        buf = np.zeros((2, *[e + 2 * h for e in ext], 3))
        inner = (slice(None),) + tuple(slice(h, h + e) for e in ext)
        sl = [slice(None)]
        for a in range(d):
            o = oracle.shard_offsets(shards[a])[idx[a]]
            sl.append(slice(o, o + ext[a]))
        buf[inner] = x[tuple(sl)]
        bufs[idx] = buf
    pos = 0
    for idx in oracle.shard_grid(shards):
        for delta in oracle.halo_directions(d):
            nb = tuple(idx[a] + delta[a] for a in range(d))
            if any(nb[a] < 0 or nb[a] >= counts[a] for a in range(d)):
                continue
            pos += (-pos) % 2            # 16-byte alignment == 2 float64
            dst = [slice(None)]
            shape = [2]
            for a in range(d):
                e = shards[a][nb[a]]
                if delta[a] == 1:        # neighbour is above: fills its low margin
                    dst.append(slice(0, h)); shape.append(h)
                elif delta[a] == -1:
                    dst.append(slice(h + e, 2 * h + e)); shape.append(h)
                else:
                    dst.append(slice(h, h + e)); shape.append(e)
            shape.append(3)
            cnt = int(np.prod(shape))
            bufs[nb][tuple(dst)] = msg[pos:pos + cnt].reshape(shape)
            pos += cnt
    assert pos == len(msg)
    for idx in oracle.shard_grid(shards):
        assert np.array_equal(bufs[idx], oracle.padded_shard(x, shards, idx, h))


def test_halo_message_counts():
    # workload topologies: number of boxes sent
    expect = {"vol32_c4to8_k3_fp32": 2, "img2048_c64_k3_bf16": 6, "vol256_c32_k3_bf16": 56,
              "vol512_c16_k5_bf16": 14, "grid1024x1792_c256_k3_bf16": 2}
    for name, n in expect.items():
        wl = synth.workload(name)
        counts = [len(s) for s in wl.shards]
        boxes = 0
        for idx in oracle.shard_grid(wl.shards):
            for delta in oracle.halo_directions(wl.ndim):
                nb = [idx[a] + delta[a] for a in range(wl.ndim)]
                boxes += all(0 <= nb[a] < counts[a] for a in range(wl.ndim))
        assert boxes == n, name


# ------------------------------------------------------- planted mistakes

def _mutants():
    def conv_flipped(x, w, b=None):
        return oracle.conv_same(x, np.flip(w, axis=tuple(range(2, w.ndim))).copy(), b)

    def conv_transposed_w(x, w, b=None):
        if w.shape[0] != w.shape[1]:
            return oracle.conv_same(x, w, b) * (1 + 1e-9)
        return oracle.conv_same(x, np.swapaxes(w, 0, 1).copy(), b)

    def conv_dropped_tap(x, w, b=None):
        w2 = w.copy()
        w2[(slice(None), slice(None)) + (0,) * (w.ndim - 2)] = 0
        return oracle.conv_same(x, w2, b)

    def conv_wrap_padding(x, w, b=None):
        k = w.shape[2]
        p = k // 2
        xp = np.pad(x, [(0, 0)] + [(p, p)] * (x.ndim - 2) + [(0, 0)], mode="wrap")
        return oracle.conv_valid(xp, w, b)

    def conv_no_bias(x, w, b=None):
        return oracle.conv_same(x, w, None)

    def gn_unbiased(y, g, eps, gamma=None, beta=None):
        mean, var = oracle.group_moments(y, g)
        m = y.size // (y.shape[0] * g)
        return oracle.group_norm_apply(y, g, mean, var * m / (m - 1), eps, gamma, beta)

    def gn_eps_outside(y, g, eps, gamma=None, beta=None):
        mean, var = oracle.group_moments(y, g)
        z = oracle.group_norm_apply(y, g, mean, var, 0.0) * np.sqrt(var.mean() / (var.mean() + eps))
        z = z * (1 if gamma is None else gamma) + (0 if beta is None else beta)
        return z

    def gn_strided_groups(y, g, eps, gamma=None, beta=None):
        c = y.shape[-1]
        perm = np.arange(c).reshape(c // g, g).T.reshape(-1)   # channel c -> group c % g
        inv = np.argsort(perm)
        z = oracle.group_norm(y[..., perm], g, eps)[..., inv]
        z = z * (1 if gamma is None else gamma) + (0 if beta is None else beta)
        return z

    good_c, good_g = oracle.conv_same, oracle.group_norm
    return {
        "flipped kernel": (conv_flipped, good_g),
        "transposed weight": (conv_transposed_w, good_g),
        "dropped tap": (conv_dropped_tap, good_g),
        "wrap padding": (conv_wrap_padding, good_g),
        "bias ignored": (conv_no_bias, good_g),
        "unbiased variance": (good_c, gn_unbiased),
        "eps outside sqrt": (good_c, gn_eps_outside),
        "strided groups": (good_c, gn_strided_groups),
    }


@pytest.mark.parametrize("name", list(_mutants()))
def test_pins_catch_mutants(name):
    conv, gn = _mutants()[name]
    results = [
        pin_bruteforce(conv, gn),
        pin_identity(conv),
        pin_shift(conv),
        pin_torch(conv, gn),
        pin_groupnorm_closed_forms(gn),
    ]
    assert not all(results), f"no pin caught the mutant '{name}'"


# ---------------------------------------------------------------- widen


def _bf16_patterns():
    """Every finite bf16 bit pattern: normals, subnormals, +-0 (exponent 0xFF,
    i.e. Inf and NaN, left out)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> np.uint16(7)) & np.uint16(0xFF)) != 0xFF
    return bits[finite]


def _pin_widen_bf16(widen_fn) -> bool:
    """widen(bits, 'bf16') against torch's own bfloat16 -> float64 conversion
    (an independent implementation) over every finite pattern, plus values
    fixed by the bf16 format: 0x3F80 = 1, 0xC000 = -2, 0x0001 = 2^-133 (the
    smallest subnormal), 0x8000 = -0.0, 0x7F7F = (2 - 2^-7) * 2^127."""
    bits = _bf16_patterns()
    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = widen_fn(bits, "bf16")
    if got.dtype != np.float64 or not np.array_equal(got.view(np.uint64), want.view(np.uint64)):
        return False
    fixed = {0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127}
    for b, v in fixed.items():
        if widen_fn(np.array([b], np.uint16), "bf16")[0] != v:
            return False
    neg0 = widen_fn(np.array([0x8000], np.uint16), "bf16")[0]
    return neg0 == 0.0 and np.signbit(neg0)


def test_widen_bf16_matches_torch_on_every_finite_pattern():
    assert _pin_widen_bf16(oracle.widen)


def test_widen_f32_is_exact():
    """fp32 -> fp64 is exact: the value survives the round trip bit for bit,
    subnormals and -0.0 included."""
    r = np.random.default_rng(3)
    a = np.concatenate([r.integers(0, 1 << 32, 100000, dtype=np.uint64).astype(np.uint32),
                        np.array([0x80000000, 0x00000001, 0x007FFFFF], np.uint32)]).view(np.float32)
    a = a[np.isfinite(a)]
    w = oracle.widen(a, "f32")
    assert w.dtype == np.float64
    assert np.array_equal(w.astype(np.float32).view(np.uint32), a.view(np.uint32))


@pytest.mark.parametrize("name", ["byte-swapped", "shift 15", "low half", "rounded via fp16"])
def test_widen_bf16_pin_catches_mutants(name):
    def byte_swapped(a, dtype):
        return (a.byteswap().astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)

    def shift15(a, dtype):
        return (a.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)

    def low_half(a, dtype):
        return a.astype(np.uint32).view(np.float32).astype(np.float64)

    def via_fp16(a, dtype):
        return a.view(np.float16).astype(np.float64)

    mutant = {"byte-swapped": byte_swapped, "shift 15": shift15, "low half": low_half,
              "rounded via fp16": via_fp16}[name]
    assert not _pin_widen_bf16(mutant), f"the widen pin did not catch the mutant '{name}'"
