"""st_groupnorm_sharded_noalloc: GroupNorm with the library's static scratch.

For callers that cannot allocate (HIP graph capture, tight serving loops).
Its output must be the same bits as st_groupnorm_sharded with a caller-owned
workspace (same kernels), on two calls in a row with the second on a smaller
input, and within the fp32 tolerance of the fp64 oracle.  An oversized request
is refused on the host before any GPU call.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from halo_sharded_conv_amd.layer import ShardedConvGN
from helpers import TOL, oracle_forward, rel_err, say, torch_bits_equal

pytestmark = pytest.mark.gpu


def _layer(wl, affine_seed, fuse_max):
    x, w = synth.make_input(wl), synth.make_weight(wl)
    gamma, beta = synth.make_affine(wl, seed=affine_seed)
    layer = ShardedConvGN(wl, fuse_max=fuse_max)
    layer.set_weight(w)
    layer.set_affine(gamma, beta)
    layer.load_input(x)
    layer.exchange()
    layer.conv()
    torch.cuda.synchronize()
    return layer, x, w, gamma, beta


def _check_case(gpu_lib, wl, affine_seed, fuse_max):
    say(f"noalloc GroupNorm: {wl.name} shards={wl.shards} batch={wl.batch} fuse_max={fuse_max}")
    layer, x, w, gamma, beta = _layer(wl, affine_seed, fuse_max)
    ymax = layer.ymax if fuse_max else None
    # the existing entry point with its own workspace
    gpu_lib.st_groupnorm_sharded(layer.out_plan, layer.y_bufs, ymax, wl.groups, wl.eps, layer.gamma, layer.beta,
                                 layer.z_bufs, layer.ws)
    z_ws = [z.clone() for z in layer.z_bufs]
    # the no-allocation entry point into fresh outputs (poisoned first)
    z_na = [torch.full_like(z, float("nan")) for z in layer.z_bufs]
    gpu_lib.st_groupnorm_sharded_noalloc(layer.out_plan, layer.y_bufs, ymax, wl.groups, wl.eps, layer.gamma,
                                         layer.beta, z_na)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(z_ws, z_na)):
        assert torch_bits_equal(a, b), f"shard {i}: noalloc output differs from the workspace entry point"
    _, z_ref = oracle_forward(wl, x, w, None, gamma, beta)
    err = rel_err(layer.gather(z_na), z_ref)
    say(f"  bitwise equal to st_groupnorm_sharded; max|err|/rms(z) vs oracle = {err:.3e}")
    assert err <= TOL[wl.dtype]


def test_noalloc_matches_workspace_entry_point_twice(gpu_lib):
    """Two calls in a row; the second on a smaller input (fewer shards, fewer
    groups, a smaller volume), so stale scratch from the first call would
    show."""
    W = synth.WORKLOADS
    big = synth.small_variant(W["img2048_c64_k3_bf16"], (37, 70), ((11, 7, 9, 10), (70,)), batch=2)
    small = synth.small_variant(W["vol32_c4to8_k3_fp32"], (9, 10, 11), ((5, 4), (10,), (11,)))
    _check_case(gpu_lib, big, affine_seed=11, fuse_max=True)
    _check_case(gpu_lib, small, affine_seed=12, fuse_max=False)


def test_noalloc_rejects_oversized_request(gpu_lib):
    """A workspace above the static scratch is refused on the host."""
    # 80 x 1024 channels: the per-channel coefficients alone take 1.25 MiB
    plan = gpu_lib.st_plan_shards(2, 80, 1024, (4, 4), ((2, 2), (4,)), (0, 0), "f32")
    need = gpu_lib.st_groupnorm_workspace_bytes(plan, 1)
    assert need > (1 << 20)
    nulls = (ctypes.c_void_p * 2)()
    st = gpu_lib.lib.st_groupnorm_sharded_noalloc(plan.handle, nulls, None, 1, ctypes.c_float(1e-5), None, None,
                                                  nulls, None)
    assert st == 5, gpu_lib.lib.st_last_error().decode()
    assert "scratch" in gpu_lib.lib.st_last_error().decode()
