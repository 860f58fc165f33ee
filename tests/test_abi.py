"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host with the documented status codes (CPU only: no call
here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import halo_sharded_conv_amd as hsc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "shardconv.h")

OK, INVALID, BAD_SHAPE, TOO_SMALL, UNSUPPORTED, WORKSPACE, HIP, ALIGN = range(8)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(st_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["st_plan_shards", "st_halo_pack", "st_halo_unpack", "st_conv_sharded",
              "st_groupnorm_sharded"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(hsc.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_status_strings():
    assert "gfx950" in hsc.st_version()
    for s in range(8):
        assert hsc.lib.st_status_string(s)


def _plan_raw(ndim, batch, ch, spatial, counts, sizes, halo, dtype=1):
    out = ctypes.c_void_p()
    sp = (ctypes.c_int64 * 3)(*spatial)
    ct = (ctypes.c_int32 * 3)(*counts)
    sz = (ctypes.c_int64 * max(1, len(sizes)))(*sizes)
    hl = (ctypes.c_int32 * 3)(*halo)
    st = hsc.lib.st_plan_shards(ndim, batch, ch, sp, ct, sz, hl, dtype, ctypes.byref(out))
    return st, out


@pytest.mark.parametrize("args,status,text", [
    ((1, 1, 4, [8, 0, 0], [1, 0, 0], [8], [1, 0, 0]), UNSUPPORTED, "ndim"),
    ((4, 1, 4, [8, 8, 8], [1, 1, 1], [8, 8, 8], [1, 1, 1]), UNSUPPORTED, "ndim"),
    ((2, 0, 4, [8, 8, 0], [1, 1, 0], [8, 8], [1, 1, 0]), INVALID, "batch"),
    ((2, 1, 0, [8, 8, 0], [1, 1, 0], [8, 8], [1, 1, 0]), INVALID, "channels"),
    ((2, 1, 4, [8, 8, 0], [2, 1, 0], [3, 4, 8], [1, 1, 0]), BAD_SHAPE, "sum"),
    ((2, 1, 4, [8, 8, 0], [2, 1, 0], [7, 1, 8], [2, 2, 0]), TOO_SMALL, "halo"),
    ((2, 1, 4, [8, 8, 0], [2, 1, 0], [8, 0, 8], [1, 1, 0]), BAD_SHAPE, "size"),
    ((2, 1, 4, [8, 8, 0], [1, 1, 0], [8, 8], [-1, 1, 0]), INVALID, "halo"),
    ((2, 1, 4, [8, 8, 0], [0, 1, 0], [8], [1, 1, 0]), INVALID, "count"),
    ((3, 1, 4, [65, 1, 1], [65, 1, 1], [1] * 65 + [1, 1], [0, 0, 0]), UNSUPPORTED, "ST_MAX_SHARDS"),
])
def test_plan_errors(args, status, text):
    st, out = _plan_raw(*args)
    assert st == status
    assert not out.value
    assert text.lower() in hsc.lib.st_last_error().decode().lower()


def test_plan_null_and_dtype_errors():
    out = ctypes.c_void_p()
    assert hsc.lib.st_plan_shards(2, 1, 4, None, None, None, None, 1, ctypes.byref(out)) == INVALID
    assert hsc.lib.st_plan_shards(2, 1, 4, None, None, None, None, 1, None) == INVALID
    st, _ = _plan_raw(2, 1, 4, [8, 8, 0], [1, 1, 0], [8, 8], [1, 1, 0], dtype=7)
    assert st == INVALID
    assert hsc.lib.st_plan_destroy(None) == INVALID
    assert hsc.lib.st_plan_num_shards(None) == -1
    assert hsc.lib.st_plan_msg_bytes(None) == -1


def test_single_shard_thinner_than_halo_is_allowed():
    # the halo only needs neighbour cells along split axes
    p = hsc.st_plan_shards(2, 1, 4, [1, 8], [[1], [8]], [2, 2], "f32")
    assert p.num_shards == 1 and p.num_halo_boxes == 0 and p.num_zero_boxes == 8


def test_python_errors_raise():
    with pytest.raises(hsc.ShardConvError) as e:
        hsc.st_plan_shards(2, 1, 4, [8, 8], [[3, 4], [8]], [1, 1], "bf16")
    assert e.value.status == BAD_SHAPE


def test_device_calls_reject_bad_arguments_before_any_launch():
    p = hsc.st_plan_shards(2, 1, 8, [8, 8], [[4, 4], [8]], [1, 1], "bf16")
    q = hsc.st_plan_shards(2, 1, 16, [8, 8], [[4, 4], [8]], [0, 0], "f32")
    q_bad = hsc.st_plan_shards(2, 1, 16, [8, 8], [[3, 5], [8]], [0, 0], "f32")
    L = hsc.lib
    PP = ctypes.c_void_p * 2
    aligned = PP(0x10000, 0x20000)
    misaligned = PP(0x10000, 0x20004)
    nulls = PP(0, 0)
    s = None
    # halo
    assert L.st_halo_pack(None, aligned, ctypes.c_void_p(0x30000), s) == INVALID
    assert L.st_halo_pack(p.handle, None, ctypes.c_void_p(0x30000), s) == INVALID
    assert L.st_halo_pack(p.handle, nulls, ctypes.c_void_p(0x30000), s) == INVALID
    assert L.st_halo_pack(p.handle, misaligned, ctypes.c_void_p(0x30000), s) == ALIGN
    assert L.st_halo_pack(p.handle, aligned, None, s) == INVALID
    assert L.st_halo_pack(p.handle, aligned, ctypes.c_void_p(0x30008), s) == ALIGN
    assert L.st_halo_unpack(p.handle, None, aligned, 1, s) == INVALID
    assert L.st_halo_unpack(p.handle, ctypes.c_void_p(0x30008), aligned, 1, s) == ALIGN
    assert L.st_halo_exchange(None, aligned, 1, s) == INVALID
    assert L.st_halo_exchange(p.handle, None, 1, s) == INVALID
    assert L.st_halo_exchange(p.handle, nulls, 1, s) == INVALID
    assert L.st_halo_exchange(p.handle, misaligned, 1, s) == ALIGN
    overlapping = PP(0x10000, 0x10010)   # padded shards are 6 x 10 x 8 bf16 = 960 bytes
    assert L.st_halo_exchange(p.handle, overlapping, 1, s) == INVALID
    assert "overlap" in hsc.lib.st_last_error().decode()
    # conv: raw weights plus a workspace (the packed weights)
    w = ctypes.c_void_p(0x40000)
    cws = ctypes.c_void_p(0xD0000)
    cneed = L.st_conv_workspace_bytes(p.handle, 16, 3)
    assert cneed >= L.st_conv_weight_bytes(2, 8, 16, 3, 1) and cneed % 256 == 0
    assert L.st_conv_workspace_bytes(p.handle, 16, 2) == 0 and L.st_conv_workspace_bytes(None, 16, 3) == 0
    cv = L.st_conv_sharded
    assert cv(p.handle, aligned, w, None, 16, 2, aligned, None, 1, cws, cneed, s) == UNSUPPORTED
    assert cv(p.handle, aligned, w, None, 16, 5, aligned, None, 1, cws, cneed, s) == BAD_SHAPE    # halo 1 < 2
    assert cv(p.handle, aligned, w, None, 16, 3, aligned, ctypes.c_void_p(0x50000), 3, cws, cneed, s) == INVALID
    assert cv(p.handle, aligned, ctypes.c_void_p(0x40008), None, 16, 3, aligned, None, 1, cws, cneed, s) == ALIGN
    assert cv(p.handle, misaligned, w, None, 16, 3, aligned, None, 1, cws, cneed, s) == ALIGN
    assert cv(p.handle, aligned, w, None, 16, 3, misaligned, None, 1, cws, cneed, s) == ALIGN
    assert cv(p.handle, nulls, w, None, 16, 3, aligned, None, 1, cws, cneed, s) == INVALID
    assert cv(None, aligned, w, None, 16, 3, aligned, None, 1, cws, cneed, s) == INVALID
    assert cv(p.handle, aligned, None, None, 16, 3, aligned, None, 1, cws, cneed, s) == INVALID
    assert cv(p.handle, aligned, w, None, 16, 3, aligned, None, 1, cws, cneed - 1, s) == WORKSPACE
    assert cv(p.handle, aligned, w, None, 16, 3, aligned, None, 1, None, cneed, s) == WORKSPACE
    assert cv(p.handle, aligned, w, None, 16, 3, aligned, None, 1, ctypes.c_void_p(0xD0008), cneed, s) == ALIGN
    cp = L.st_conv_sharded_packed
    assert cp(p.handle, aligned, w, None, 16, 2, aligned, None, 1, s) == UNSUPPORTED
    assert cp(p.handle, aligned, w, None, 16, 5, aligned, None, 1, s) == BAD_SHAPE
    assert cp(p.handle, aligned, ctypes.c_void_p(0x40008), None, 16, 3, aligned, None, 1, s) == ALIGN
    assert cp(None, aligned, w, None, 16, 3, aligned, None, 1, s) == INVALID
    # weights
    assert L.st_conv_weight_bytes(2, 8, 16, 2, 1) == 0
    assert L.st_conv_weight_bytes(4, 8, 16, 3, 1) == 0
    assert L.st_conv_weight_bytes(2, 8, 16, 3, 9) == 0
    assert L.st_conv_pack_weights(2, 8, 16, 4, 1, w, w, s) == UNSUPPORTED
    assert L.st_conv_pack_weights(2, 8, 16, 3, 1, None, w, s) == INVALID
    assert L.st_conv_pack_weights(2, 8, 16, 3, 1, ctypes.c_void_p(0x40002), w, s) == ALIGN
    w2 = ctypes.c_void_p(0x48000)
    assert L.st_conv_dgrad_weights(4, 8, 16, 3, 1, w, w2, s) == UNSUPPORTED
    assert L.st_conv_dgrad_weights(2, 8, 16, 2, 1, w, w2, s) == UNSUPPORTED
    assert L.st_conv_dgrad_weights(2, 8, 16, 3, 9, w, w2, s) == UNSUPPORTED
    assert L.st_conv_dgrad_weights(2, 8, 16, 3, 1, None, w2, s) == INVALID
    assert L.st_conv_dgrad_weights(2, 8, 16, 3, 1, w, w, s) == INVALID
    # groupnorm
    need = L.st_groupnorm_workspace_bytes(q.handle, 4)
    assert need > 0
    ws = ctypes.c_void_p(0x60000)
    gn = L.st_groupnorm_sharded
    assert gn(q.handle, aligned, None, 4, 1e-5, None, None, aligned, ws, need - 1, s) == WORKSPACE
    assert gn(q.handle, aligned, None, 4, 1e-5, None, None, aligned, None, need, s) == WORKSPACE
    assert gn(q.handle, aligned, None, 5, 1e-5, None, None, aligned, ws, need, s) == INVALID
    assert gn(q.handle, aligned, None, 4, -1.0, None, None, aligned, ws, need, s) == INVALID
    assert gn(p.handle, aligned, None, 4, 1e-5, None, None, aligned, ws, need, s) == BAD_SHAPE
    assert gn(q.handle, misaligned, None, 4, 1e-5, None, None, aligned, ws, need, s) == ALIGN
    assert gn(q.handle, aligned, None, 4, 1e-5, None, None, aligned, ctypes.c_void_p(0x60008), need, s) == ALIGN
    assert gn(q.handle, aligned, ctypes.c_void_p(0x70002), 4, 1e-5, None, None, aligned, ws, need, s) == ALIGN
    # weight gradient
    qd = hsc.st_plan_shards(2, 1, 16, [8, 8], [[4, 4], [8]], [1, 1], "bf16")      # dy, any halo
    need_w = L.st_conv_wgrad_workspace_bytes(p.handle, 16, 3)
    assert need_w > 0 and L.st_conv_wgrad_workspace_bytes(p.handle, 16, 2) == 0
    dw = ctypes.c_void_p(0xB0000)
    wws = ctypes.c_void_p(0xC0000)
    wg = L.st_conv_wgrad
    assert wg(None, aligned, qd.handle, aligned, 3, dw, wws, need_w, s) == INVALID
    assert wg(p.handle, aligned, qd.handle, aligned, 3, None, wws, need_w, s) == INVALID
    assert wg(p.handle, aligned, qd.handle, aligned, 4, dw, wws, need_w, s) == UNSUPPORTED
    assert wg(p.handle, aligned, qd.handle, aligned, 5, dw, wws, need_w, s) == BAD_SHAPE     # halo 1 < 2
    assert wg(p.handle, aligned, q.handle, aligned, 3, dw, wws, need_w, s) == BAD_SHAPE      # dtype differs
    assert wg(p.handle, aligned, q_bad.handle, aligned, 3, dw, wws, need_w, s) == BAD_SHAPE
    assert wg(p.handle, aligned, qd.handle, aligned, 3, dw, wws, need_w - 1, s) == WORKSPACE
    assert wg(p.handle, aligned, qd.handle, aligned, 3, dw, None, need_w, s) == WORKSPACE
    assert wg(p.handle, misaligned, qd.handle, aligned, 3, dw, wws, need_w, s) == ALIGN
    assert wg(p.handle, aligned, qd.handle, nulls, 3, dw, wws, need_w, s) == INVALID
    assert wg(p.handle, aligned, qd.handle, aligned, 3, ctypes.c_void_p(0xB0004), wws, need_w, s) == ALIGN
    # pooling: derived plan and its errors
    pp = hsc.st_plan_shards(2, 1, 16, [8, 8], [[1, 1, 6], [8]], [1, 1], "bf16")
    out = ctypes.c_void_p()
    assert L.st_plan_pooled(pp.handle, 2, 2, None, 1, ctypes.byref(out)) == TOO_SMALL   # shard 1 holds no window start
    assert L.st_plan_pooled(p.handle, 9, 2, None, 1, ctypes.byref(out)) == BAD_SHAPE     # window larger than the volume
    assert L.st_plan_pooled(p.handle, 2, 0, None, 1, ctypes.byref(out)) == INVALID
    assert L.st_plan_pooled(None, 2, 2, None, 1, ctypes.byref(out)) == INVALID
    pq = hsc.st_plan_pooled(p, 2, 2)
    assert pq.shards == ((2, 2), (4,))
    assert L.st_pool_sharded(p.handle, aligned, 2, 2, 2, pq.handle, aligned, s) == INVALID   # mode
    assert L.st_pool_sharded(p.handle, aligned, 3, 2, 0, pq.handle, aligned, s) == BAD_SHAPE  # not its pooled plan
    assert L.st_pool_sharded(p.handle, misaligned, 2, 2, 0, pq.handle, aligned, s) == ALIGN
    p0 = hsc.st_plan_shards(2, 1, 8, [8, 8], [[4, 4], [8]], [0, 0], "bf16")                # no halo
    pq0 = hsc.st_plan_pooled(p0, 3, 2)
    assert L.st_pool_sharded(p0.handle, aligned, 3, 2, 0, pq0.handle, aligned, s) == BAD_SHAPE
    # strided conv: derived plan and its errors
    assert L.st_plan_strided(pp.handle, 3, 2, 8, None, ctypes.byref(out)) == TOO_SMALL    # a shard holds no centre
    assert L.st_plan_strided(p.handle, 4, 2, 8, None, ctypes.byref(out)) == UNSUPPORTED
    assert L.st_plan_strided(p.handle, 3, 0, 8, None, ctypes.byref(out)) == INVALID
    sq = hsc.st_plan_strided(p, 3, 2, 16)
    assert sq.shards == ((2, 2), (4,)) and sq.channels == 16
    wt = ctypes.c_void_p(0xF0000)
    tws = ctypes.c_void_p(0xE0000)
    sneed = L.st_conv_strided_workspace_bytes(p.handle, 16, 3)
    assert sneed == -(-9 * 8 * 16 * 4 // 256) * 256
    assert L.st_conv_strided_workspace_bytes(p.handle, 16, 4) == 0
    cs = L.st_conv_strided_sharded
    assert cs(p.handle, aligned, None, None, 3, 2, sq.handle, aligned, tws, sneed, s) == INVALID
    assert cs(p.handle, aligned, wt, None, 3, 3, sq.handle, aligned, tws, sneed, s) == BAD_SHAPE   # not its plan
    assert cs(p.handle, aligned, wt, None, 2, 2, sq.handle, aligned, tws, sneed, s) == UNSUPPORTED
    assert cs(p.handle, misaligned, wt, None, 3, 2, sq.handle, aligned, tws, sneed, s) == ALIGN
    assert cs(p.handle, aligned, wt, None, 3, 2, p.handle, aligned, tws, sneed, s) == BAD_SHAPE     # bf16 output plan
    assert cs(p.handle, aligned, wt, None, 3, 2, sq.handle, aligned, tws, sneed - 4, s) == WORKSPACE
    assert cs(p.handle, aligned, wt, None, 3, 2, sq.handle, aligned, None, sneed, s) == WORKSPACE
    assert cs(p.handle, aligned, ctypes.c_void_p(0xF0002), None, 3, 2, sq.handle, aligned, tws, sneed, s) == ALIGN
    sq0 = hsc.st_plan_strided(p0, 3, 2, 8)
    assert cs(p0.handle, aligned, wt, None, 3, 2, sq0.handle, aligned, tws, sneed, s) == BAD_SHAPE  # halo 0 < 1
    # transposed conv: derived plan and its errors
    assert L.st_plan_transposed(p.handle, 4, 2, 8, None, ctypes.byref(out)) == UNSUPPORTED
    assert L.st_plan_transposed(p.handle, 3, 0, 8, None, ctypes.byref(out)) == INVALID
    assert L.st_plan_transposed(p.handle, 3, 9, 8, None, ctypes.byref(out)) == INVALID
    assert L.st_plan_transposed(p.handle, 3, 2, 0, None, ctypes.byref(out)) == INVALID
    tq = hsc.st_plan_transposed(p, 3, 2, 16)
    assert tq.shards == ((8, 8), (16,)) and tq.channels == 16
    tneed = L.st_conv_transposed_workspace_bytes(p.handle, 16, 7)
    ct = L.st_conv_transposed_sharded
    assert ct(p.handle, aligned, None, None, 3, 2, tq.handle, aligned, tws, tneed, s) == INVALID
    assert ct(p.handle, aligned, wt, None, 3, 3, tq.handle, aligned, tws, tneed, s) == BAD_SHAPE   # not its plan
    assert ct(p.handle, aligned, wt, None, 2, 2, tq.handle, aligned, tws, tneed, s) == UNSUPPORTED
    assert ct(p.handle, misaligned, wt, None, 3, 2, tq.handle, aligned, tws, tneed, s) == ALIGN
    assert ct(p.handle, aligned, ctypes.c_void_p(0xF0002), None, 3, 2, tq.handle, aligned, tws, tneed, s) == ALIGN
    assert ct(p.handle, aligned, wt, None, 3, 2, p.handle, aligned, tws, tneed, s) == BAD_SHAPE     # bf16 output plan
    assert ct(p.handle, nulls, wt, None, 3, 2, tq.handle, aligned, tws, tneed, s) == INVALID
    assert ct(p.handle, aligned, wt, None, 3, 2, tq.handle, aligned, None, tneed, s) == WORKSPACE
    tq0 = hsc.st_plan_transposed(p0, 3, 2, 8)
    assert ct(p0.handle, aligned, wt, None, 3, 2, tq0.handle, aligned, tws, tneed, s) == BAD_SHAPE  # halo 0 < 1
    tq7 = hsc.st_plan_transposed(p, 7, 2, 16)      # k 7, stride 2 reads cells q-1 .. q+2
    assert ct(p.handle, aligned, wt, None, 7, 2, tq7.handle, aligned, tws, tneed, s) == BAD_SHAPE   # halo 1 < 2
    # groupnorm backward
    bneed = L.st_groupnorm_backward_workspace_bytes(q.handle, 4)
    assert bneed > 0 and L.st_groupnorm_backward_workspace_bytes(None, 4) == 0
    bws = ctypes.c_void_p(0x80000)
    dzs = PP(0x90000, 0xA0000)
    gb = L.st_groupnorm_backward
    args = [q.handle, aligned, dzs, None, None, 4, None, ws, need, None, aligned, None, None, bws, bneed, s]

    def gbw(**kw):
        a = list(args)
        names = ["plan", "y", "dz", "ymax", "dzmax", "groups", "gamma", "fws", "fnb", "dyplan", "dy", "dg", "db",
                 "ws", "nb", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return gb(*a)
    assert gbw(plan=None) == INVALID
    assert gbw(dz=None) == INVALID
    assert gbw(dz=nulls) == INVALID
    assert gbw(dz=misaligned) == ALIGN
    assert gbw(dy=misaligned) == ALIGN
    assert gbw(groups=5) == INVALID
    assert gbw(fnb=need - 1) == WORKSPACE
    assert gbw(fws=None) == WORKSPACE
    assert gbw(nb=bneed - 1) == WORKSPACE
    assert gbw(ws=None) == WORKSPACE
    assert gbw(ws=ctypes.c_void_p(0x80008)) == ALIGN
    assert gbw(ws=ws, nb=max(need, bneed)) == INVALID
    assert gbw(dzmax=ctypes.c_void_p(0x70002)) == ALIGN
    assert gbw(dg=ctypes.c_void_p(0x70002)) == ALIGN
    assert gbw(plan=p.handle) == BAD_SHAPE
    # dy in another layout: same shards and channels, bf16 needs C % 4 == 0, no aliasing
    dyp_ok = hsc.st_plan_shards(2, 1, 16, [8, 8], [[4, 4], [8]], [1, 1], "bf16")
    dyp_ch = hsc.st_plan_shards(2, 1, 8, [8, 8], [[4, 4], [8]], [1, 1], "bf16")
    dyp_sh = hsc.st_plan_shards(2, 1, 16, [8, 8], [[3, 5], [8]], [1, 1], "bf16")
    dys = PP(0xD0000, 0xE0000)
    assert gbw(dyplan=dyp_ch.handle, dy=dys) == BAD_SHAPE
    assert gbw(dyplan=dyp_sh.handle, dy=dys) == BAD_SHAPE
    assert gbw(dyplan=dyp_ok.handle, dy=aligned) == INVALID          # dy aliases y
    assert gbw(dyplan=dyp_ok.handle, dy=PP(0xD0000, 0xE0008)) == ALIGN
    assert gbw(dyplan=dyp_ok.handle, dy=PP(0xD0000, 0)) == INVALID


def test_workspace_layout_regions_are_disjoint():
    q = hsc.st_plan_shards(3, 2, 32, [6, 7, 8], [[3, 3], [7], [4, 4]], [0, 0, 0], "f32")
    lay = hsc.st_groupnorm_workspace_layout(q, 8)
    S, N, G, C = 4, 2, 8, 32
    regions = sorted([
        (lay["partials_offset"], S * N * G * 16), (lay["ymax_offset"], N * G * 4),
        (lay["stats_offset"], N * G * 8), (lay["scales_offset"], N * G * 8),
        (lay["chan_offset"], N * C * 16)])
    for (o1, n1), (o2, _) in zip(regions, regions[1:]):
        assert o1 + n1 <= o2
    assert regions[-1][0] + regions[-1][1] <= lay["total_bytes"]
    assert hsc.st_groupnorm_workspace_bytes(q, 8) == lay["total_bytes"]
    with pytest.raises(hsc.ShardConvError):
        hsc.st_groupnorm_workspace_layout(q, 5)


def test_one_hip_runtime_in_process():
    """The binding must share torch's HIP runtime: a second runtime in the
    process would see torch's streams and allocations as foreign objects."""
    import subprocess
    import sys
    code = ("import halo_sharded_conv_amd as h, torch;"
            "print(len(h._hip_runtimes()))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "1"
