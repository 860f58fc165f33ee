"""Random shard plans (seeded): any uneven plan is a correct plan, and the
method's invariant says the result must not depend on it.

For each drawn case (one of the matrix-core layer shapes or the fp32 layer, a
random volume with ragged extents, 1-3 shards per axis with random uneven
sizes no thinner than the halo): the forward y and z equal the unsharded run
bit for bit and meet the oracle's tolerance; the GroupNorm backward's dy,
dgamma and dbeta equal the unsharded run bit for bit; the weight gradient
meets the oracle's tolerance.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from halo_sharded_conv_amd.layer import ShardedConvGN
from helpers import TOL, bits_equal, oracle_forward, rel_err, say

pytestmark = pytest.mark.gpu

BASES = ["img2048_c64_k3_bf16", "vol256_c32_k3_bf16", "vol512_c16_k5_bf16", "vol32_c4to8_k3_fp32",
         "grid1024x1792_c256_k3_bf16"]


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    base = synth.workload(BASES[seed % len(BASES)])
    h = base.ksize // 2
    if base.ndim == 2:
        c = base.cin
        spatial = (int(rng.integers(8, 48)), int(rng.integers(8, 160 if c < 256 else 40)))
    else:
        spatial = tuple(int(v) for v in rng.integers(6, 22, size=3))
    shards = []
    for n in spatial:
        parts = int(rng.integers(1, 4))
        while parts > 1 and n < parts * max(h, 1):
            parts -= 1
        shards.append(tuple(synth.shard_sizes(n, parts, max(h, 1), None, rng)))
    batch = int(rng.integers(1, 3))
    return dataclasses.replace(base, name=f"{base.name}_rand{seed}", spatial=spatial, shards=tuple(shards),
                               batch=batch)


def forward(wl, x, w, gamma, beta, dz):
    layer = ShardedConvGN(wl)
    layer.set_weight(w)
    layer.set_affine(gamma, beta)
    layer.load_input(x)
    layer.step()
    layer.alloc_backward()
    layer.load_upstream_grad(dz)
    layer.norm_backward()
    torch.cuda.synchronize()
    return layer


@pytest.mark.parametrize("seed", range(10))
def test_random_plan(seed):
    wl = draw(seed)
    say(f"random plan {seed}: {wl.name} N={wl.batch} spatial={wl.spatial} shards={wl.shards}")
    x, w = synth.make_input(wl), synth.make_weight(wl)
    gamma, beta = synth.make_affine(wl, seed=seed)
    dz = synth.make_upstream_grad(wl, seed=seed + 7)
    a = forward(wl, x, w, gamma, beta, dz)
    b = forward(wl.unsharded(), x, w, gamma, beta, dz)
    assert bits_equal(a.y_host(), b.y_host()) and bits_equal(a.z_host(), b.z_host())
    assert bits_equal(a.gather(a.dy_bufs), b.gather(b.dy_bufs))
    assert bits_equal(a.dgamma.cpu().numpy(), b.dgamma.cpu().numpy())
    assert bits_equal(a.dbeta.cpu().numpy(), b.dbeta.cpu().numpy())
    y_ref, z_ref = oracle_forward(wl, x, w, None, gamma, beta)
    ey, ez = rel_err(a.y_host(), y_ref), rel_err(a.z_host(), z_ref)
    say(f"  max|err|/rms y {ey:.2e} z {ez:.2e}")
    assert ey <= TOL[wl.dtype] and ez <= TOL[wl.dtype]
