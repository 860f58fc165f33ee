"""Planner geometry against the oracle's halo definitions (CPU only).

The library's box table is replayed with numpy copies (pack = sender box ->
message, unpack = message -> receiver margin, zero boxes -> zeros); the
message bytes must equal the oracle's halo message and every rebuilt padded
shard must equal the oracle's padded shard.  Planner queries are host-only.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st_

import halo_sharded_conv_amd as hsc
import oracle
import synth


def replay(plan, x, shards, h, C, esize):
    d = len(shards)
    N = x.shape[0]
    bufs = []
    for i in range(plan.num_shards):
        inf = plan.shard_info(i)
        b = np.full((N, *inf["padded"], C), np.nan if x.dtype.kind == "f" else 0x7FFF, dtype=x.dtype)
        src = [slice(None)] + [slice(o, o + e) for o, e in zip(inf["offset"], inf["extent"])]
        dst = [slice(None)] + [slice(h, h + e) for e in inf["extent"]]
        b[tuple(dst)] = x[tuple(src)]
        bufs.append(b)
    msg = np.zeros(plan.msg_bytes, np.uint8)
    nreal = plan.num_halo_boxes
    boxes = [plan.halo_box(i) for i in range(nreal + plan.num_zero_boxes)]
    for b in boxes[:nreal]:
        sl = [slice(None)] + [slice(lo, lo + e) for lo, e in zip(b["src_lo"], b["ext"])]
        data = np.ascontiguousarray(bufs[b["src"]][tuple(sl)]).view(np.uint8).reshape(-1)
        msg[b["msg_offset"]:b["msg_offset"] + data.size] = data
    out = [bb.copy() for bb in bufs]
    cover = [np.zeros(bb.shape[:-1], np.int32) for bb in bufs]
    for b in boxes:
        sl = tuple([slice(None)] + [slice(lo, lo + e) for lo, e in zip(b["dst_lo"], b["ext"])])
        shape = out[b["dst"]][sl].shape
        if b["src"] >= 0:
            cnt = int(np.prod(shape)) * esize
            out[b["dst"]][sl] = msg[b["msg_offset"]:b["msg_offset"] + cnt].view(x.dtype).reshape(shape)
        else:
            out[b["dst"]][sl] = 0
        cover[b["dst"]][sl] += 1
    return msg, out, cover, boxes


def check_plan(shards, h, C, dtype, N=1, seed=0):
    d = len(shards)
    spatial = [sum(s) for s in shards]
    rng = np.random.default_rng(seed)
    if dtype == "f32":
        x = rng.standard_normal((N, *spatial, C)).astype(np.float32)
        esize = 4
    else:
        x = rng.integers(0, 2 ** 16, size=(N, *spatial, C), dtype=np.uint16)
        esize = 2
    plan = hsc.st_plan_shards(d, N, C, spatial, shards, [h] * d, dtype)
    assert plan.num_shards == math.prod(len(s) for s in shards)
    for i, idx in enumerate(oracle.shard_grid(shards)):
        inf = plan.shard_info(i)
        assert inf["grid"] == idx
        assert inf["offset"] == tuple(oracle.shard_offsets(shards[a])[idx[a]] for a in range(d))
        assert inf["extent"] == tuple(shards[a][idx[a]] for a in range(d))
        assert inf["padded"] == tuple(e + 2 * h for e in inf["extent"])
        assert inf["elems"] == N * math.prod(inf["padded"]) * C
        assert inf["bytes"] == inf["elems"] * esize
    msg, out, cover, boxes = replay(plan, x, shards, h, C, esize)
    want = np.frombuffer(oracle.halo_message(x, shards, h), np.uint8)
    assert plan.msg_bytes == want.size
    assert np.array_equal(msg, want)
    for i, idx in enumerate(oracle.shard_grid(shards)):
        ref = oracle.padded_shard(x, shards, idx, h)
        assert np.array_equal(out[i].view(np.uint8), ref.view(np.uint8))
        # margins covered exactly once, interior never
        inner = tuple(slice(h, h + e) for e in plan.shard_info(i)["extent"])
        c = cover[i].copy()
        assert np.all(c[(slice(None),) + inner] == 0)
        c[(slice(None),) + inner] = 1
        assert np.all(c == 1)
    return plan


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_topologies(name):
    wl = synth.workload(name)
    # same shard grid on a small volume keeps the replay cheap
    small = [tuple(max(wl.halo, 1) + (i % 3) + 2 for i in range(len(s))) for s in wl.shards]
    plan = check_plan(small, wl.halo, 8 if wl.dtype == "bf16" else 4, wl.dtype)
    expect = {"vol32_c4to8_k3_fp32": 2, "img2048_c64_k3_bf16": 6, "vol256_c32_k3_bf16": 56,
              "vol512_c16_k5_bf16": 14, "grid1024x1792_c256_k3_bf16": 2}[name]
    assert plan.num_halo_boxes == expect
    assert plan.num_halo_boxes + plan.num_zero_boxes == wl.num_shards * (3 ** wl.ndim - 1)


def test_full_size_message_sizes():
    # payload bytes of the workloads' halos, from the plan alone
    expect = {"vol32_c4to8_k3_fp32": 2 * 32 * 32 * 4 * 4,
              "img2048_c64_k3_bf16": 6 * 2048 * 64 * 2,
              "vol512_c16_k5_bf16": 14 * 2 * 512 * 512 * 16 * 2,
              "grid1024x1792_c256_k3_bf16": 2 * 1024 * 256 * 2}
    for name, want in expect.items():
        wl = synth.workload(name)
        p = hsc.st_plan_shards(wl.ndim, 1, wl.cin, wl.spatial, wl.shards, [wl.halo] * wl.ndim, wl.dtype)
        assert p.msg_bytes == want, name


@pytest.mark.parametrize("shards,h,C,dtype,N", [
    (((3, 4), (5, 3)), 1, 4, "f32", 2),
    (((4, 3, 5), (6,)), 2, 6, "bf16", 1),
    (((3, 4), (2, 3), (4, 3)), 1, 8, "bf16", 2),
    (((5, 4, 6), (7,), (6,)), 2, 2, "bf16", 1),
    (((7,), (3, 3, 3)), 3, 3, "f32", 1),
    (((9,), (11,)), 1, 5, "bf16", 3),
])
def test_plans_against_oracle(shards, h, C, dtype, N):
    check_plan(shards, h, C, dtype, N)


@settings(max_examples=40, deadline=None)
@given(st_.data())
def test_random_plans(data):
    d = data.draw(st_.sampled_from([2, 3]))
    h = data.draw(st_.integers(0, 2))
    shards = []
    for _ in range(d):
        n = data.draw(st_.integers(1, 3))
        lo = max(1, h)
        shards.append(tuple(data.draw(st_.integers(lo, lo + 4)) for _ in range(n)))
    C = data.draw(st_.sampled_from([1, 2, 3, 4, 8]))
    dtype = data.draw(st_.sampled_from(["f32", "bf16"]))
    check_plan(shards, h, C, dtype, N=data.draw(st_.integers(1, 2)), seed=data.draw(st_.integers(0, 99)))


def test_halo_box_above_2_31_words_is_refused():
    # the copy kernels split a box's word index with 32-bit multiply-shift
    # division, valid below 2^31: an H-face box of 2^30 cells x 32 bytes
    # (2^31 16-byte words) is refused at plan time, one word less is planned
    import halo_sharded_conv_amd as hsc
    with pytest.raises(hsc.ShardConvError, match="halo box too large"):
        hsc.st_plan_shards(2, 1, 8, (4, 2 ** 30), ((2, 2), (2 ** 30,)), (1, 0), "f32")
    p = hsc.st_plan_shards(2, 1, 8, (4, 2 ** 30 - 1), ((2, 2), (2 ** 30 - 1,)), (1, 0), "f32")
    assert p.num_shards == 2
