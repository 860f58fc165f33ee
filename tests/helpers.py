"""Shared helpers of the GPU tests: workloads, oracle results, comparisons."""
from __future__ import annotations

import dataclasses
import math
import sys

import numpy as np

import oracle
import synth

# Tolerances on max |gpu - oracle| / rms(oracle), as the target states them:
# fp32 operands 1e-5, bf16 operands (fp32 accumulation, fp32 outputs) 1e-2.
TOL = {"f32": 1e-5, "bf16": 1e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, want) -> float:
    want = np.asarray(want, np.float64)
    rms = math.sqrt(float(np.mean(want * want)))
    return float(np.max(np.abs(np.asarray(got, np.float64) - want))) / max(rms, 1e-300)


def small_cases():
    """Small versions of every workload: same channels, kernel, groups and
    dtype; shard topologies like the full ones; extents that leave ragged
    tails against every conv tile shape; some with batch 2."""
    W = synth.WORKLOADS
    return {
        "vol32_full": W["vol32_c4to8_k3_fp32"],
        "vol32_b2": synth.small_variant(W["vol32_c4to8_k3_fp32"], (9, 10, 11), ((5, 4), (10,), (11,)), batch=2),
        "img64_small": synth.small_variant(W["img2048_c64_k3_bf16"], (37, 70), ((11, 7, 9, 10), (70,))),
        "img64_b2": synth.small_variant(W["img2048_c64_k3_bf16"], (20, 130), ((8, 12), (130,)), batch=2),
        "vol32_grid": synth.small_variant(W["vol256_c32_k3_bf16"], (9, 19, 37), ((4, 5), (11, 8), (17, 20))),
        "vol16k5": synth.small_variant(W["vol512_c16_k5_bf16"], (23, 13, 40), ((2, 5, 3, 4, 2, 3, 2, 2), (13,), (40,))),
        # two samples, shards deeper than one 8-plane step of the k5 kernel
        "vol16k5_b2": synth.small_variant(W["vol512_c16_k5_bf16"], (21, 9, 33), ((9, 12), (9,), (33,)), batch=2),
        "grid256_small": synth.small_variant(W["grid1024x1792_c256_k3_bf16"], (5, 150), ((5,), (80, 70))),
    }


def direct_cases():
    """bf16 shapes without a tuned kernel: channel counts off the matrix-core
    grid (the direct kernel) and on it (the matrix-core implicit GEMM of the
    strided conv at stride 1, with max |y| in a pass of its own)."""
    base = synth.WORKLOADS["img2048_c64_k3_bf16"]
    vol = synth.WORKLOADS["vol512_c16_k5_bf16"]
    a = dataclasses.replace(base, name="img_c5to12_k3", cin=5, cout=12, groups=3, spatial=(13, 17),
                            shards=((6, 7), (9, 8)))
    b = dataclasses.replace(vol, name="vol_c3to4_k5", cin=3, cout=4,
                            groups=2, spatial=(7, 8, 9), shards=((3, 4), (8,), (2, 7)))
    c = dataclasses.replace(base, name="img_c48to80_k3", cin=48, cout=80, groups=5, spatial=(19, 70),
                            shards=((7, 12), (33, 37)), batch=2)
    d = dataclasses.replace(synth.WORKLOADS["vol256_c32_k3_bf16"], name="vol_c128to128_k3", cin=128, cout=128,
                            groups=8, spatial=(9, 10, 11), shards=((4, 5), (10,), (6, 5)))
    e = dataclasses.replace(base, name="img_c32to48_k5", cin=32, cout=48, groups=3, ksize=5, spatial=(17, 40),
                            shards=((8, 9), (21, 19)))
    # channel counts that are not multiples of 4: one-channel vectors in the
    # GroupNorm kernels, 4-byte halo words, one bf16 channel per conv load
    f = dataclasses.replace(base, name="img_c6to10_k3", cin=6, cout=10, groups=5, spatial=(15, 37),
                            shards=((7, 8), (20, 17)))
    return {"img_c5to12_k3": a, "vol_c3to4_k5": b, "img_c48to80_k3": c, "vol_c128to128_k3": d,
            "img_c32to48_k5": e, "img_c6to10_k3": f}


def oracle_forward(wl, x, w, bias=None, gamma=None, beta=None):
    """fp64 y and z of the unsharded definition."""
    xf = oracle.widen(x, wl.dtype)
    wf = oracle.widen(w, wl.dtype)
    y = oracle.conv_same(xf, wf, bias)
    z = oracle.group_norm(y, wl.groups, wl.eps, gamma, beta)
    return y, z


def bits_equal(a, b) -> bool:
    return np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))


def torch_bits_equal(t1, t2) -> bool:
    import torch
    return bool(torch.equal(t1.view(torch.int32), t2.view(torch.int32)))


def dev_raw(a):
    """A host array as a GPU tensor of the same bits (bf16 patterns stay
    uint16 bit patterns, viewed as int16): what the library is handed."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a.reshape(-1).copy()).cuda()


def dev_workspace(nbytes: int):
    import torch
    return torch.empty(max(16, int(nbytes)), dtype=torch.uint8, device="cuda")
