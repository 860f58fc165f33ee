"""The seeded input module: determinism, bf16 rounding, shard-size rules (CPU)."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    a = np.concatenate([
        r.standard_normal(100000).astype(np.float32) * np.float32(10) ** r.integers(-30, 30, 100000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-40, -1e-42], np.float32),
        # exact ties: mantissa low half == 0x8000, both parities of bit 16
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ]).astype(np.float32)
    a = a[np.isfinite(a)]
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(a), want)


def test_shard_vectors_reproduce():
    wl = synth.WORKLOADS
    assert wl["vol32_c4to8_k3_fp32"].shards[0] == (17, 15)
    assert wl["img2048_c64_k3_bf16"].shards[0] == (1034, 298, 322, 394)
    assert wl["vol256_c32_k3_bf16"].shards == ((126, 130), (121, 135), (137, 119))
    assert wl["vol512_c16_k5_bf16"].shards[0] == (66, 79, 71, 60, 62, 59, 54, 61)
    assert wl["grid1024x1792_c256_k3_bf16"].shards[1] == (900, 892)


def test_shard_sizes_properties():
    for seed in range(200):
        r = np.random.default_rng(seed)
        total = int(r.integers(50, 5000))
        parts = int(r.integers(1, 9))
        lo = int(r.integers(1, max(2, total // parts)))
        avg = total // parts
        hi = None if seed % 2 else max(lo, avg) + avg // 2 + 1
        s = synth.shard_sizes(total, parts, lo, hi, np.random.default_rng(seed))
        assert sum(s) == total and len(s) == parts
        assert min(s) >= lo and (hi is None or max(s) <= hi)


def test_workload_table_consistent():
    for wl in synth.WORKLOADS.values():
        assert len(wl.shards) == wl.ndim == len(wl.spatial)
        for ax, s in enumerate(wl.shards):
            assert sum(s) == wl.spatial[ax] and min(s) >= wl.halo
        assert wl.cout % wl.groups == 0 and wl.ksize % 2 == 1


def test_inputs_deterministic_and_shaped():
    base = synth.workload("grid1024x1792_c256_k3_bf16")
    wl = synth.small_variant(base, (6, 10), ((6,), (4, 6)))
    a, b = synth.make_input(wl), synth.make_input(wl)
    assert a.dtype == np.uint16 and a.shape == (1, 6, 10, 256)
    assert np.array_equal(a, b)
    w = synth.make_weight(wl)
    assert w.shape == (256, 256, 3, 3) and w.dtype == np.uint16
    f = synth.workload("vol32_c4to8_k3_fp32")
    x = synth.make_input(f)
    assert x.dtype == np.float32 and x.shape == (1, 32, 32, 32, 4)
    assert abs(float(x.mean())) < 0.02 and abs(float(x.std()) - 1) < 0.02
    wf = synth.make_weight(f)
    assert np.all(np.abs(wf) <= 1 / np.sqrt(108))


def test_sample_positions_cover_seams():
    wl = synth.workload("vol256_c32_k3_bf16")
    pos = synth.sample_positions(wl, 500, 0)
    assert pos.shape[1] == 4 and len(pos) >= 500
    for ax in range(3):
        s = wl.shards[ax][0]
        vals = set(pos[:, 1 + ax].tolist())
        assert {s - 2, s - 1, s, s + 1} <= vals
    assert np.all(pos[:, 1:] < np.array(wl.spatial)) and np.all(pos >= 0)
