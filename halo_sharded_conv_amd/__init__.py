"""Python binding of libshardconv (the halo-sharded conv + GroupNorm library).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch tensors supply device memory and the current stream.  The
binding fails loudly if the library is missing or a tensor is not on a GPU;
there is no CPU fallback.

Names match the C-ABI in include/shardconv.h (st_plan_shards, st_halo_pack,
st_halo_unpack, st_conv_sharded, st_groupnorm_sharded, ...).
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libshardconv.so")

ST_F32, ST_BF16 = 0, 1
ST_MAX_SHARDS = 64
DTYPES = {"f32": ST_F32, "bf16": ST_BF16}
ESIZE = {ST_F32: 4, ST_BF16: 2}


class ShardConvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class _ShardInfo(ctypes.Structure):
    _fields_ = [("index", ctypes.c_int32), ("grid", ctypes.c_int32 * 3),
                ("offset", ctypes.c_int64 * 3), ("extent", ctypes.c_int64 * 3),
                ("padded", ctypes.c_int64 * 3), ("elems", ctypes.c_int64),
                ("bytes", ctypes.c_int64)]


class _HaloBox(ctypes.Structure):
    _fields_ = [("src_shard", ctypes.c_int32), ("dst_shard", ctypes.c_int32),
                ("dir", ctypes.c_int32 * 3), ("dst_lo", ctypes.c_int64 * 3),
                ("src_lo", ctypes.c_int64 * 3), ("ext", ctypes.c_int64 * 3),
                ("msg_offset", ctypes.c_int64)]


class _GnLayout(ctypes.Structure):
    _fields_ = [("partials_offset", ctypes.c_size_t), ("stats_offset", ctypes.c_size_t),
                ("scales_offset", ctypes.c_size_t), ("ymax_offset", ctypes.c_size_t),
                ("chan_offset", ctypes.c_size_t), ("total_bytes", ctypes.c_size_t)]


def _hip_runtimes() -> list:
    """Paths of every HIP runtime library mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python halo_sharded_conv_amd/build.py`")
    # torch ships its own HIP runtime and its libraries ask for it by a name
    # that does not match an already loaded libamdhip64.so.7.  Loading torch
    # first lets this library bind to torch's runtime (same soname), so
    # torch's streams and allocations and these kernels share one runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    runtimes = _hip_runtimes()
    if len(runtimes) > 1:
        raise ImportError(f"two HIP runtimes are loaded ({runtimes}); import torch before any other HIP library")
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    PP = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "st_version": (ctypes.c_char_p, []),
        "st_last_error": (ctypes.c_char_p, []),
        "st_status_string": (ctypes.c_char_p, [I32]),
        "st_plan_shards": (I32, [I32, I64, I64, ctypes.POINTER(I64), ctypes.POINTER(I32),
                                 ctypes.POINTER(I64), ctypes.POINTER(I32), I32, ctypes.POINTER(P)]),
        "st_plan_destroy": (I32, [P]),
        "st_plan_num_shards": (I64, [P]),
        "st_plan_msg_bytes": (I64, [P]),
        "st_plan_num_halo_boxes": (I64, [P]),
        "st_plan_num_zero_boxes": (I64, [P]),
        "st_plan_upload": (I32, [P, P]),
        "st_plan_shard_info": (I32, [P, I32, ctypes.POINTER(_ShardInfo)]),
        "st_plan_halo_box": (I32, [P, I32, ctypes.POINTER(_HaloBox)]),
        "st_halo_pack": (I32, [P, PP, P, P]),
        "st_halo_unpack": (I32, [P, P, PP, I32, P]),
        "st_halo_exchange": (I32, [P, PP, I32, P]),
        "st_conv_weight_bytes": (SZ, [I32, I32, I32, I32, I32]),
        "st_conv_pack_weights": (I32, [I32, I32, I32, I32, I32, P, P, P]),
        "st_conv_dgrad_weights": (I32, [I32, I32, I32, I32, I32, P, P, P]),
        "st_conv_workspace_bytes": (SZ, [P, I32, I32]),
        "st_conv_sharded": (I32, [P, PP, P, P, I32, I32, PP, P, I32, P, SZ, P]),
        "st_conv_sharded_packed": (I32, [P, PP, P, P, I32, I32, PP, P, I32, P]),
        "st_plan_pooled": (I32, [P, I32, I32, ctypes.POINTER(I32), I32, ctypes.POINTER(P)]),
        "st_pool_sharded": (I32, [P, PP, I32, I32, I32, P, PP, P]),
        "st_plan_strided": (I32, [P, I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(P)]),
        "st_conv_strided_workspace_bytes": (SZ, [P, I32, I32]),
        "st_conv_strided_sharded": (I32, [P, PP, P, P, I32, I32, P, PP, P, SZ, P]),
        "st_plan_transposed": (I32, [P, I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(P)]),
        "st_conv_transposed_workspace_bytes": (SZ, [P, I32, I32]),
        "st_conv_transposed_sharded": (I32, [P, PP, P, P, I32, I32, P, PP, P, SZ, P]),
        "st_conv_wgrad_workspace_bytes": (SZ, [P, I32, I32]),
        "st_conv_wgrad": (I32, [P, PP, P, PP, I32, P, P, SZ, P]),
        "st_groupnorm_workspace_bytes": (SZ, [P, I32]),
        "st_groupnorm_workspace_layout": (I32, [P, I32, ctypes.POINTER(_GnLayout)]),
        "st_groupnorm_sharded": (I32, [P, PP, P, I32, ctypes.c_float, P, P, PP, P, SZ, P]),
        "st_groupnorm_sharded_noalloc": (I32, [P, PP, P, I32, ctypes.c_float, P, P, PP, P]),
        "st_groupnorm_partials": (I32, [P, PP, P, I32, P, SZ, P]),
        "st_groupnorm_combine": (I32, [P, I32, ctypes.c_float, P, P, P, SZ, P]),
        "st_groupnorm_apply": (I32, [P, PP, I32, PP, P, SZ, P]),
        "st_groupnorm_combine_apply": (I32, [P, PP, I32, ctypes.c_float, P, P, PP, P, SZ, P]),
        "st_groupnorm_backward_workspace_bytes": (SZ, [P, I32]),
        "st_groupnorm_backward": (I32, [P, PP, PP, P, P, I32, P, P, SZ, P, PP, P, P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib.st_last_error().decode()
        name = lib.st_status_string(status).decode()
        raise ShardConvError(status, f"{what}: {name}: {msg}")


def st_version() -> str:
    return lib.st_version().decode()


# ---------------------------------------------------------------- plans

class Plan:
    """Owns an st_plan*; released on destroy() or garbage collection."""

    def __init__(self, handle: int, ndim: int, batch: int, channels: int, dtype: int,
                 shards: Sequence[Sequence[int]], halo: Sequence[int]):
        self._h = ctypes.c_void_p(handle)
        self.ndim, self.batch, self.channels, self.dtype = ndim, batch, channels, dtype
        self.shards = tuple(tuple(s) for s in shards)
        self.halo = tuple(halo)

    @property
    def handle(self) -> ctypes.c_void_p:
        if not self._h:
            raise ShardConvError(1, "plan already destroyed")
        return self._h

    def destroy(self) -> None:
        if self._h:
            _check(lib.st_plan_destroy(self._h), "st_plan_destroy")
            self._h = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    @property
    def num_shards(self) -> int:
        return int(lib.st_plan_num_shards(self.handle))

    @property
    def msg_bytes(self) -> int:
        return int(lib.st_plan_msg_bytes(self.handle))

    @property
    def num_halo_boxes(self) -> int:
        return int(lib.st_plan_num_halo_boxes(self.handle))

    @property
    def num_zero_boxes(self) -> int:
        return int(lib.st_plan_num_zero_boxes(self.handle))

    def upload(self, stream=None) -> None:
        """Put the halo descriptor table on the current device now (needed
        before a graph capture that contains the plan's first halo call)."""
        _check(lib.st_plan_upload(self.handle, _stream(stream)), "st_plan_upload")

    def shard_info(self, i: int) -> dict:
        info = _ShardInfo()
        _check(lib.st_plan_shard_info(self.handle, i, ctypes.byref(info)), "st_plan_shard_info")
        d = self.ndim
        return {"index": info.index, "grid": tuple(info.grid[:d]), "offset": tuple(info.offset[:d]),
                "extent": tuple(info.extent[:d]), "padded": tuple(info.padded[:d]),
                "elems": info.elems, "bytes": info.bytes}

    def padded_shape(self, i: int) -> tuple:
        return (self.batch, *self.shard_info(i)["padded"], self.channels)

    def halo_box(self, i: int) -> dict:
        b = _HaloBox()
        _check(lib.st_plan_halo_box(self.handle, i, ctypes.byref(b)), "st_plan_halo_box")
        d = self.ndim
        return {"src": b.src_shard, "dst": b.dst_shard, "dir": tuple(b.dir[:d]),
                "dst_lo": tuple(b.dst_lo[:d]), "src_lo": tuple(b.src_lo[:d]),
                "ext": tuple(b.ext[:d]), "msg_offset": b.msg_offset}


def st_plan_shards(ndim: int, batch: int, channels: int, spatial: Sequence[int],
                   shard_sizes: Sequence[Sequence[int]], halo: Sequence[int], dtype) -> Plan:
    """Plan over per-axis shard sizes (axis 0 outermost); dtype 'f32'/'bf16' or 0/1."""
    dt = DTYPES.get(dtype, dtype)
    n_axes = len(spatial)
    sp = (ctypes.c_int64 * max(1, n_axes))(*spatial)
    counts = (ctypes.c_int32 * max(1, len(shard_sizes)))(*[len(s) for s in shard_sizes])
    flat = [int(v) for s in shard_sizes for v in s]
    sizes = (ctypes.c_int64 * max(1, len(flat)))(*flat)
    hl = (ctypes.c_int32 * max(1, len(halo)))(*halo)
    out = ctypes.c_void_p()
    _check(lib.st_plan_shards(ndim, batch, channels, sp, counts, sizes, hl, dt, ctypes.byref(out)),
           "st_plan_shards")
    return Plan(out.value, ndim, batch, channels, dt, shard_sizes, halo)


# ------------------------------------------------------------ device calls

def _torch():
    import torch
    return torch


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev_ptr(t, what: str, min_bytes: int = 0) -> int:
    if t is None:
        return 0
    if not getattr(t, "is_cuda", False):
        raise ShardConvError(1, f"{what}: expected a GPU tensor (no CPU fallback exists)")
    if not t.is_contiguous():
        raise ShardConvError(1, f"{what}: tensor must be contiguous")
    nbytes = t.numel() * t.element_size()
    if nbytes < min_bytes:
        raise ShardConvError(2, f"{what}: tensor holds {nbytes} bytes, needs {min_bytes}")
    return t.data_ptr()


def _ptr_array(tensors, what: str, sizes: List[int]):
    if len(tensors) != len(sizes):
        raise ShardConvError(2, f"{what}: expected {len(sizes)} shard buffers, got {len(tensors)}")
    arr = (ctypes.c_void_p * max(1, len(tensors)))()
    for i, t in enumerate(tensors):
        arr[i] = _dev_ptr(t, f"{what}[{i}]", sizes[i])
    return arr


def _shard_bytes(plan: Plan) -> List[int]:
    return [plan.shard_info(i)["bytes"] for i in range(plan.num_shards)]


def st_halo_pack(plan: Plan, shard_bufs, msg, stream=None) -> None:
    arr = _ptr_array(shard_bufs, "st_halo_pack shard", _shard_bytes(plan))
    m = _dev_ptr(msg, "st_halo_pack msg", plan.msg_bytes) if plan.msg_bytes else 0
    _check(lib.st_halo_pack(plan.handle, arr, ctypes.c_void_p(m), _stream(stream)), "st_halo_pack")


def st_halo_unpack(plan: Plan, msg, shard_bufs, zero_global_margins: bool = True, stream=None) -> None:
    arr = _ptr_array(shard_bufs, "st_halo_unpack shard", _shard_bytes(plan))
    m = _dev_ptr(msg, "st_halo_unpack msg", plan.msg_bytes) if plan.msg_bytes else 0
    _check(lib.st_halo_unpack(plan.handle, ctypes.c_void_p(m), arr, int(bool(zero_global_margins)),
                              _stream(stream)), "st_halo_unpack")



def st_halo_exchange(plan: Plan, shard_bufs, zero_global_margins: bool = True, stream=None) -> None:
    arr = _ptr_array(shard_bufs, "st_halo_exchange shard", _shard_bytes(plan))
    _check(lib.st_halo_exchange(plan.handle, arr, int(bool(zero_global_margins)), _stream(stream)),
           "st_halo_exchange")

def st_conv_weight_bytes(ndim: int, cin: int, cout: int, ksize: int, dtype) -> int:
    return int(lib.st_conv_weight_bytes(ndim, cin, cout, ksize, DTYPES.get(dtype, dtype)))


def st_conv_pack_weights(ndim: int, cin: int, cout: int, ksize: int, dtype, weight, packed,
                         stream=None) -> None:
    dt = DTYPES.get(dtype, dtype)
    need = st_conv_weight_bytes(ndim, cin, cout, ksize, dt)
    raw = cout * cin * ksize ** ndim * ESIZE[dt]
    _check(lib.st_conv_pack_weights(ndim, cin, cout, ksize, dt,
                                    ctypes.c_void_p(_dev_ptr(weight, "weight", raw)),
                                    ctypes.c_void_p(_dev_ptr(packed, "packed weight", need)),
                                    _stream(stream)), "st_conv_pack_weights")


def st_conv_dgrad_weights(ndim: int, cin: int, cout: int, ksize: int, dtype, weight, out,
                          stream=None) -> None:
    dt = DTYPES.get(dtype, dtype)
    raw = cout * cin * ksize ** ndim * ESIZE[dt]
    _check(lib.st_conv_dgrad_weights(ndim, cin, cout, ksize, dt,
                                     ctypes.c_void_p(_dev_ptr(weight, "weight", raw)),
                                     ctypes.c_void_p(_dev_ptr(out, "dgrad weight", raw)),
                                     _stream(stream)), "st_conv_dgrad_weights")


def _y_bytes(in_plan: Plan, cout: int) -> List[int]:
    """Bytes of each shard's unpadded fp32 conv output [N][extent...][cout]."""
    out = []
    for i in range(in_plan.num_shards):
        n = in_plan.batch * cout * 4
        for e in in_plan.shard_info(i)["extent"]:
            n *= e
        out.append(n)
    return out


def st_conv_workspace_bytes(in_plan: Plan, cout: int, ksize: int) -> int:
    return int(lib.st_conv_workspace_bytes(in_plan.handle, cout, ksize))


def st_conv_sharded(in_plan: Plan, in_bufs, weight, bias, cout: int, ksize: int, y_bufs, ymax=None,
                    groups: int = 1, workspace=None, stream=None) -> None:
    """weight: raw [Cout][Cin][k..] in the plan's dtype (bf16 as int16/uint16
    bits); workspace: >= st_conv_workspace_bytes bytes."""
    ins = _ptr_array(in_bufs, "st_conv_sharded input", _shard_bytes(in_plan))
    outs = _ptr_array(y_bufs, "st_conv_sharded y", _y_bytes(in_plan, cout))
    raw = cout * in_plan.channels * ksize ** in_plan.ndim * ESIZE[in_plan.dtype]
    w = _dev_ptr(weight, "weight", raw)
    b = _dev_ptr(bias, "bias", 4 * cout)
    ym = _dev_ptr(ymax, "ymax", 4 * in_plan.batch * groups) if ymax is not None else 0
    ws, nb = _ws(workspace)
    _check(lib.st_conv_sharded(in_plan.handle, ins, ctypes.c_void_p(w), ctypes.c_void_p(b), cout, ksize, outs,
                               ctypes.c_void_p(ym), groups, ctypes.c_void_p(ws), nb, _stream(stream)),
           "st_conv_sharded")


def st_conv_sharded_packed(in_plan: Plan, in_bufs, packed_weight, bias, cout: int, ksize: int, y_bufs, ymax=None,
                           groups: int = 1, stream=None) -> None:
    """packed_weight: from st_conv_pack_weights."""
    ins = _ptr_array(in_bufs, "st_conv_sharded_packed input", _shard_bytes(in_plan))
    outs = _ptr_array(y_bufs, "st_conv_sharded_packed y", _y_bytes(in_plan, cout))
    need_w = st_conv_weight_bytes(in_plan.ndim, in_plan.channels, cout, ksize, in_plan.dtype)
    w = _dev_ptr(packed_weight, "packed weight", need_w)
    b = _dev_ptr(bias, "bias", 4 * cout)
    ym = _dev_ptr(ymax, "ymax", 4 * in_plan.batch * groups) if ymax is not None else 0
    _check(lib.st_conv_sharded_packed(in_plan.handle, ins, ctypes.c_void_p(w), ctypes.c_void_p(b), cout, ksize,
                                      outs, ctypes.c_void_p(ym), groups, _stream(stream)),
           "st_conv_sharded_packed")


def st_plan_pooled(in_plan: Plan, ksize: int, stride: int, out_halo=None, out_dtype=None) -> Plan:
    """Output plan of a 'valid' pooling; its shard sizes are derived by the library."""
    dt = in_plan.dtype if out_dtype is None else DTYPES.get(out_dtype, out_dtype)
    hl = (ctypes.c_int32 * 3)(*(list(out_halo) + [0] * (3 - len(out_halo)))) if out_halo is not None else None
    out = ctypes.c_void_p()
    _check(lib.st_plan_pooled(in_plan.handle, ksize, stride, hl, dt, ctypes.byref(out)), "st_plan_pooled")
    halo = tuple(out_halo) if out_halo is not None else (0,) * in_plan.ndim
    probe = Plan(out.value, in_plan.ndim, in_plan.batch, in_plan.channels, dt, (), halo)
    # per-axis shard sizes from the shard table (shards are row-major over the grid)
    n = probe.num_shards
    infos = [probe.shard_info(i) for i in range(n)]
    sizes = []
    for a in range(in_plan.ndim):
        seen = {}
        for inf in infos:
            seen.setdefault(inf["grid"][a], inf["extent"][a])
        sizes.append(tuple(seen[g] for g in sorted(seen)))
    probe.shards = tuple(sizes)
    return probe


def st_pool_sharded(in_plan: Plan, in_bufs, ksize: int, stride: int, mode: str, out_plan: Plan, out_bufs,
                    stream=None) -> None:
    """mode 'avg' or 'max'."""
    ins = _ptr_array(in_bufs, "st_pool_sharded input", _shard_bytes(in_plan))
    outs = _ptr_array(out_bufs, "st_pool_sharded output", _shard_bytes(out_plan))
    m = {"avg": 0, "max": 1}[mode]
    _check(lib.st_pool_sharded(in_plan.handle, ins, ksize, stride, m, out_plan.handle, outs, _stream(stream)),
           "st_pool_sharded")


def _plan_from_handle(handle, ndim, batch, channels, dtype, halo) -> Plan:
    """Wrap a library-derived plan, recovering its per-axis shard sizes."""
    plan = Plan(handle, ndim, batch, channels, dtype, (), halo)
    infos = [plan.shard_info(i) for i in range(plan.num_shards)]
    sizes = []
    for a in range(ndim):
        seen = {}
        for inf in infos:
            seen.setdefault(inf["grid"][a], inf["extent"][a])
        sizes.append(tuple(seen[g] for g in sorted(seen)))
    plan.shards = tuple(sizes)
    return plan


def st_plan_strided(in_plan: Plan, ksize: int, stride: int, cout: int, out_halo=None) -> Plan:
    """fp32 output plan of a strided 'same'-padded conv; shard sizes derived by the library."""
    hl = (ctypes.c_int32 * 3)(*(list(out_halo) + [0] * (3 - len(out_halo)))) if out_halo is not None else None
    out = ctypes.c_void_p()
    _check(lib.st_plan_strided(in_plan.handle, ksize, stride, cout, hl, ctypes.byref(out)), "st_plan_strided")
    return _plan_from_handle(out.value, in_plan.ndim, in_plan.batch, cout, ST_F32,
                             tuple(out_halo) if out_halo is not None else (0,) * in_plan.ndim)


def st_conv_strided_workspace_bytes(in_plan: Plan, cout: int, ksize: int) -> int:
    return int(lib.st_conv_strided_workspace_bytes(in_plan.handle, cout, ksize))


def st_conv_strided_sharded(in_plan: Plan, in_bufs, weight, bias, ksize: int, stride: int, out_plan: Plan,
                            out_bufs, workspace, stream=None) -> None:
    """weight: raw [Cout][Cin][k..] in the input plan's dtype."""
    ins = _ptr_array(in_bufs, "st_conv_strided_sharded input", _shard_bytes(in_plan))
    outs = _ptr_array(out_bufs, "st_conv_strided_sharded output", _shard_bytes(out_plan))
    taps = ksize ** in_plan.ndim
    w = _dev_ptr(weight, "weight", ESIZE[in_plan.dtype] * taps * in_plan.channels * out_plan.channels)
    b = _dev_ptr(bias, "bias", 4 * out_plan.channels)
    ws, nb = _ws(workspace)
    _check(lib.st_conv_strided_sharded(in_plan.handle, ins, ctypes.c_void_p(w), ctypes.c_void_p(b), ksize, stride,
                                       out_plan.handle, outs, ctypes.c_void_p(ws), nb, _stream(stream)),
           "st_conv_strided_sharded")


def st_plan_transposed(in_plan: Plan, ksize: int, stride: int, cout: int, out_halo=None) -> Plan:
    """fp32 output plan of a transposed (upsampling) conv: every shard's extents times stride."""
    hl = (ctypes.c_int32 * 3)(*(list(out_halo) + [0] * (3 - len(out_halo)))) if out_halo is not None else None
    out = ctypes.c_void_p()
    _check(lib.st_plan_transposed(in_plan.handle, ksize, stride, cout, hl, ctypes.byref(out)), "st_plan_transposed")
    return _plan_from_handle(out.value, in_plan.ndim, in_plan.batch, cout, ST_F32,
                             tuple(out_halo) if out_halo is not None else (0,) * in_plan.ndim)


def st_conv_transposed_workspace_bytes(in_plan: Plan, cout: int, ksize: int) -> int:
    return int(lib.st_conv_transposed_workspace_bytes(in_plan.handle, cout, ksize))


def st_conv_transposed_sharded(in_plan: Plan, in_bufs, weight, bias, ksize: int, stride: int, out_plan: Plan,
                               out_bufs, workspace, stream=None) -> None:
    """weight: raw [Cin][Cout][k..] (Cin = in_plan.channels) in the input plan's dtype."""
    ins = _ptr_array(in_bufs, "st_conv_transposed_sharded input", _shard_bytes(in_plan))
    outs = _ptr_array(out_bufs, "st_conv_transposed_sharded output", _shard_bytes(out_plan))
    taps = ksize ** in_plan.ndim
    w = _dev_ptr(weight, "weight", ESIZE[in_plan.dtype] * taps * in_plan.channels * out_plan.channels)
    b = _dev_ptr(bias, "bias", 4 * out_plan.channels)
    ws, nb = _ws(workspace)
    _check(lib.st_conv_transposed_sharded(in_plan.handle, ins, ctypes.c_void_p(w), ctypes.c_void_p(b), ksize,
                                          stride, out_plan.handle, outs, ctypes.c_void_p(ws), nb, _stream(stream)),
           "st_conv_transposed_sharded")


def st_conv_wgrad_workspace_bytes(x_plan: Plan, cout: int, ksize: int) -> int:
    return int(lib.st_conv_wgrad_workspace_bytes(x_plan.handle, cout, ksize))


def st_conv_wgrad(x_plan: Plan, x_bufs, dy_plan: Plan, dy_bufs, ksize: int, dweight, workspace,
                  stream=None) -> None:
    xs = _ptr_array(x_bufs, "st_conv_wgrad x", _shard_bytes(x_plan))
    dys = _ptr_array(dy_bufs, "st_conv_wgrad dy", _shard_bytes(dy_plan))
    elems = dy_plan.channels * x_plan.channels * ksize ** x_plan.ndim
    dw = _dev_ptr(dweight, "dweight", 4 * elems)
    ws, nb = _ws(workspace)
    _check(lib.st_conv_wgrad(x_plan.handle, xs, dy_plan.handle, dys, ksize, ctypes.c_void_p(dw),
                             ctypes.c_void_p(ws), nb, _stream(stream)), "st_conv_wgrad")


def st_groupnorm_workspace_bytes(y_plan: Plan, groups: int) -> int:
    return int(lib.st_groupnorm_workspace_bytes(y_plan.handle, groups))


def st_groupnorm_workspace_layout(y_plan: Plan, groups: int) -> dict:
    l = _GnLayout()
    _check(lib.st_groupnorm_workspace_layout(y_plan.handle, groups, ctypes.byref(l)),
           "st_groupnorm_workspace_layout")
    return {f: getattr(l, f) for f, _ in _GnLayout._fields_}


def st_groupnorm_sharded(y_plan: Plan, y_bufs, ymax, groups: int, eps: float, gamma, beta,
                         z_bufs, workspace, stream=None) -> None:
    sizes = _shard_bytes(y_plan)
    ys = _ptr_array(y_bufs, "st_groupnorm_sharded y", sizes)
    zs = _ptr_array(z_bufs, "st_groupnorm_sharded z", sizes)
    ym = _dev_ptr(ymax, "ymax", 4 * y_plan.batch * groups) if ymax is not None else 0
    g = _dev_ptr(gamma, "gamma", 4 * y_plan.channels)
    b = _dev_ptr(beta, "beta", 4 * y_plan.channels)
    ws = _dev_ptr(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.st_groupnorm_sharded(y_plan.handle, ys, ctypes.c_void_p(ym), groups, float(eps),
                                    ctypes.c_void_p(g), ctypes.c_void_p(b), zs, ctypes.c_void_p(ws),
                                    ws_bytes, _stream(stream)), "st_groupnorm_sharded")


def st_groupnorm_sharded_noalloc(y_plan: Plan, y_bufs, ymax, groups: int, eps: float, gamma, beta,
                                 z_bufs, stream=None) -> None:
    """st_groupnorm_sharded with the library's static scratch as workspace
    (no device allocation; calls that overlap on one GPU race)."""
    sizes = _shard_bytes(y_plan)
    ys = _ptr_array(y_bufs, "st_groupnorm_sharded_noalloc y", sizes)
    zs = _ptr_array(z_bufs, "st_groupnorm_sharded_noalloc z", sizes)
    ym = _dev_ptr(ymax, "ymax", 4 * y_plan.batch * groups) if ymax is not None else 0
    g = _dev_ptr(gamma, "gamma", 4 * y_plan.channels)
    b = _dev_ptr(beta, "beta", 4 * y_plan.channels)
    _check(lib.st_groupnorm_sharded_noalloc(y_plan.handle, ys, ctypes.c_void_p(ym), groups, float(eps),
                                            ctypes.c_void_p(g), ctypes.c_void_p(b), zs, _stream(stream)),
           "st_groupnorm_sharded_noalloc")


def _ws(workspace):
    ws = _dev_ptr(workspace, "workspace")
    return ws, (workspace.numel() * workspace.element_size() if workspace is not None else 0)


def st_groupnorm_partials(y_plan: Plan, y_bufs, ymax, groups: int, workspace, stream=None) -> None:
    ys = _ptr_array(y_bufs, "st_groupnorm_partials y", _shard_bytes(y_plan))
    ym = _dev_ptr(ymax, "ymax", 4 * y_plan.batch * groups) if ymax is not None else 0
    ws, nb = _ws(workspace)
    _check(lib.st_groupnorm_partials(y_plan.handle, ys, ctypes.c_void_p(ym), groups, ctypes.c_void_p(ws), nb,
                                     _stream(stream)), "st_groupnorm_partials")


def st_groupnorm_combine(y_plan: Plan, groups: int, eps: float, gamma, beta, workspace, stream=None) -> None:
    g = _dev_ptr(gamma, "gamma", 4 * y_plan.channels)
    b = _dev_ptr(beta, "beta", 4 * y_plan.channels)
    ws, nb = _ws(workspace)
    _check(lib.st_groupnorm_combine(y_plan.handle, groups, float(eps), ctypes.c_void_p(g), ctypes.c_void_p(b),
                                    ctypes.c_void_p(ws), nb, _stream(stream)), "st_groupnorm_combine")


def st_groupnorm_apply(y_plan: Plan, y_bufs, groups: int, z_bufs, workspace, stream=None) -> None:
    sizes = _shard_bytes(y_plan)
    ys = _ptr_array(y_bufs, "st_groupnorm_apply y", sizes)
    zs = _ptr_array(z_bufs, "st_groupnorm_apply z", sizes)
    ws, nb = _ws(workspace)
    _check(lib.st_groupnorm_apply(y_plan.handle, ys, groups, zs, ctypes.c_void_p(ws), nb, _stream(stream)),
           "st_groupnorm_apply")


def st_groupnorm_combine_apply(y_plan: Plan, y_bufs, groups: int, eps: float, gamma, beta, z_bufs, workspace,
                               stream=None) -> None:
    sizes = _shard_bytes(y_plan)
    ys = _ptr_array(y_bufs, "st_groupnorm_combine_apply y", sizes)
    zs = _ptr_array(z_bufs, "st_groupnorm_combine_apply z", sizes)
    g = _dev_ptr(gamma, "gamma", 4 * y_plan.channels)
    b = _dev_ptr(beta, "beta", 4 * y_plan.channels)
    ws, nb = _ws(workspace)
    _check(lib.st_groupnorm_combine_apply(y_plan.handle, ys, groups, float(eps), ctypes.c_void_p(g),
                                          ctypes.c_void_p(b), zs, ctypes.c_void_p(ws), nb, _stream(stream)),
           "st_groupnorm_combine_apply")


def st_groupnorm_backward_workspace_bytes(y_plan: Plan, groups: int) -> int:
    return int(lib.st_groupnorm_backward_workspace_bytes(y_plan.handle, groups))


def st_groupnorm_backward(y_plan: Plan, y_bufs, dz_bufs, ymax, dzmax, groups: int, gamma, fwd_workspace,
                          dy_bufs, dgamma, dbeta, workspace, stream=None, dy_plan: Optional[Plan] = None) -> None:
    """dy_plan None: dy in y's fp32 layout; else dy written into dy_plan's
    (padded, fp32 or bf16) shard interiors."""
    sizes = _shard_bytes(y_plan)
    ys = _ptr_array(y_bufs, "st_groupnorm_backward y", sizes)
    dzs = _ptr_array(dz_bufs, "st_groupnorm_backward dz", sizes)
    dys = _ptr_array(dy_bufs, "st_groupnorm_backward dy", sizes if dy_plan is None else _shard_bytes(dy_plan))
    ng = 4 * y_plan.batch * groups
    ym = _dev_ptr(ymax, "ymax", ng) if ymax is not None else 0
    dm = _dev_ptr(dzmax, "dzmax", ng) if dzmax is not None else 0
    g = _dev_ptr(gamma, "gamma", 4 * y_plan.channels)
    dg = _dev_ptr(dgamma, "dgamma", 4 * y_plan.channels)
    db = _dev_ptr(dbeta, "dbeta", 4 * y_plan.channels)
    fws, fnb = _ws(fwd_workspace)
    ws, nb = _ws(workspace)
    _check(lib.st_groupnorm_backward(y_plan.handle, ys, dzs, ctypes.c_void_p(ym), ctypes.c_void_p(dm), groups,
                                     ctypes.c_void_p(g), ctypes.c_void_p(fws), fnb,
                                     dy_plan.handle if dy_plan is not None else None, dys, ctypes.c_void_p(dg),
                                     ctypes.c_void_p(db), ctypes.c_void_p(ws), nb, _stream(stream)),
           "st_groupnorm_backward")


__all__ = [
    "lib", "LIB_PATH", "ShardConvError", "Plan", "ST_F32", "ST_BF16", "st_version",
    "st_plan_shards", "st_halo_pack", "st_halo_unpack", "st_halo_exchange", "st_conv_weight_bytes", "st_conv_dgrad_weights",
    "st_conv_pack_weights", "st_conv_workspace_bytes", "st_conv_sharded", "st_conv_sharded_packed",
    "st_groupnorm_workspace_bytes", "st_conv_strided_workspace_bytes", "st_conv_transposed_workspace_bytes",
    "st_groupnorm_workspace_layout", "st_groupnorm_sharded", "st_groupnorm_sharded_noalloc", "st_groupnorm_partials",
    "st_groupnorm_combine", "st_groupnorm_apply", "st_groupnorm_backward_workspace_bytes",
    "st_groupnorm_backward", "st_conv_wgrad_workspace_bytes", "st_conv_wgrad", "st_plan_pooled",
    "st_pool_sharded", "st_plan_strided", "st_conv_strided_sharded", "st_plan_transposed",
    "st_conv_transposed_sharded",
]
