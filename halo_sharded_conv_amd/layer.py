"""One domain-sharded conv + GroupNorm layer held on the GPU.

Owns the plans and every device buffer (allocated through torch) and runs the
four steps through the library: halo pack, halo unpack, per-shard conv,
split-statistics GroupNorm.  torch is used for allocation, host<->device
copies of inputs/outputs and slicing views; no arithmetic of the layer runs
outside the library's kernels.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

from . import (ST_BF16, ST_F32, ShardConvError, st_conv_dgrad_weights, st_conv_sharded,
               st_conv_workspace_bytes, st_groupnorm_apply, st_groupnorm_backward,
               st_groupnorm_backward_workspace_bytes, st_groupnorm_combine, st_groupnorm_combine_apply,
               st_groupnorm_partials,
               st_groupnorm_sharded, st_groupnorm_workspace_bytes, st_groupnorm_workspace_layout,
               st_halo_exchange, st_halo_pack, st_halo_unpack, st_plan_shards)


def _torch():
    import torch
    return torch


class ShardedConvGN:
    """Buffers and plans for one layer.

    cfg needs: ndim, batch, cin, cout, spatial, shards, ksize, groups, eps,
    dtype ('f32' or 'bf16').  Shard buffers are channels-last and padded by
    ksize//2 on every face.
    """

    def __init__(self, cfg, device: str = "cuda", alias_z: bool = False, fuse_max: bool = True):
        torch = _torch()
        if not torch.cuda.is_available():
            raise ShardConvError(6, "no GPU: the layer runs only on the HIP library")
        self.cfg = cfg
        self.device = torch.device(device)
        self.fuse_max = fuse_max
        d, h = cfg.ndim, cfg.ksize // 2
        self.h = h
        self.dtype = ST_F32 if cfg.dtype == "f32" else ST_BF16
        self.in_plan = st_plan_shards(d, cfg.batch, cfg.cin, cfg.spatial, cfg.shards, [h] * d, self.dtype)
        self.out_plan = st_plan_shards(d, cfg.batch, cfg.cout, cfg.spatial, cfg.shards, [0] * d, ST_F32)
        self.S = self.in_plan.num_shards
        self.info = [self.in_plan.shard_info(i) for i in range(self.S)]
        tdt = torch.float32 if self.dtype == ST_F32 else torch.int16
        self.x_bufs = [torch.zeros(i["elems"], dtype=tdt, device=self.device) for i in self.info]
        self.msg = torch.zeros(max(16, self.in_plan.msg_bytes), dtype=torch.uint8, device=self.device)
        wb = st_conv_workspace_bytes(self.in_plan, cfg.cout, cfg.ksize)
        if wb == 0:
            raise ShardConvError(4, "unsupported conv shape")
        # raw weights [Cout][Cin][k..] in the operand type, and the conv's
        # workspace (the weights packed for its kernel, rewritten every call)
        self.w_raw = torch.zeros(cfg.cout * cfg.cin * cfg.ksize ** d, dtype=tdt, device=self.device)
        self.conv_ws = torch.zeros(wb, dtype=torch.uint8, device=self.device)
        self.out_info = [self.out_plan.shard_info(i) for i in range(self.S)]
        self.y_bufs = [torch.empty(i["elems"], dtype=torch.float32, device=self.device) for i in self.out_info]
        self.z_bufs = self.y_bufs if alias_z else [torch.empty_like(y) for y in self.y_bufs]
        self.ymax = torch.zeros(cfg.batch * cfg.groups, dtype=torch.int32, device=self.device)
        self.ws = torch.zeros(st_groupnorm_workspace_bytes(self.out_plan, cfg.groups), dtype=torch.uint8,
                              device=self.device)
        self.bias = None
        self.gamma = None
        self.beta = None

    # ------------------------------------------------------------ inputs
    def _host_to_dev(self, a: np.ndarray):
        torch = _torch()
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(self.device)

    def set_weight(self, w: np.ndarray, bias: Optional[np.ndarray] = None) -> None:
        """w: [Cout, Cin, k..] float32 (fp32 layer) or uint16 bf16 bits."""
        self.w_raw.copy_(self._host_to_dev(w.reshape(-1)))
        self.bias = None if bias is None else self._host_to_dev(np.asarray(bias, np.float32))
        _torch().cuda.synchronize()

    def set_weight_dgrad(self, w_forward: np.ndarray) -> None:
        """For a layer built from dgrad_config(forward_cfg): its conv becomes the
        input gradient of the forward conv.  w_forward: the forward weights
        [Cout, Cin, k..] (Cout = this layer's cin); they are transposed and
        flipped on the device."""
        cfg = self.cfg
        torch = _torch()
        raw = self._host_to_dev(w_forward.reshape(-1))
        st_conv_dgrad_weights(cfg.ndim, cfg.cout, cfg.cin, cfg.ksize, self.dtype, raw, self.w_raw)
        self.bias = None
        torch.cuda.synchronize()

    def set_affine(self, gamma: Optional[np.ndarray], beta: Optional[np.ndarray]) -> None:
        self.gamma = None if gamma is None else self._host_to_dev(np.asarray(gamma, np.float32))
        self.beta = None if beta is None else self._host_to_dev(np.asarray(beta, np.float32))

    def padded_view(self, i: int):
        return self.x_bufs[i].view(self.in_plan.padded_shape(i))

    def interior_view(self, i: int):
        v = self.padded_view(i)
        h = self.h
        sl = [slice(None)] + [slice(h, h + e) for e in self.info[i]["extent"]] + [slice(None)]
        return v[tuple(sl)]

    def _global_slices(self, i: int):
        inf = self.info[i]
        return tuple([slice(None)] + [slice(o, o + e) for o, e in zip(inf["offset"], inf["extent"])])

    def load_input(self, x: np.ndarray) -> None:
        """x: channels-last [N, *spatial, Cin] (float32 or uint16 bf16 bits)."""
        for i in range(self.S):
            part = x[self._global_slices(i)]
            self.interior_view(i).copy_(self._host_to_dev(part))
        _torch().cuda.synchronize()

    # ------------------------------------------------------------- steps
    def exchange_pack(self, stream=None) -> None:
        st_halo_pack(self.in_plan, self.x_bufs, self.msg, stream)

    def exchange_unpack(self, zero_global_margins: bool = True, stream=None) -> None:
        st_halo_unpack(self.in_plan, self.msg, self.x_bufs, zero_global_margins, stream)

    def exchange(self, zero_global_margins: bool = True, stream=None) -> None:
        st_halo_pack(self.in_plan, self.x_bufs, self.msg, stream)
        st_halo_unpack(self.in_plan, self.msg, self.x_bufs, zero_global_margins, stream)

    def exchange_fused(self, zero_global_margins: bool = True, stream=None) -> None:
        st_halo_exchange(self.in_plan, self.x_bufs, zero_global_margins, stream)

    def conv(self, stream=None) -> None:
        cfg = self.cfg
        st_conv_sharded(self.in_plan, self.x_bufs, self.w_raw, self.bias, cfg.cout, cfg.ksize, self.y_bufs,
                        self.ymax if self.fuse_max else None, cfg.groups, self.conv_ws, stream)

    def norm(self, stream=None) -> None:
        cfg = self.cfg
        st_groupnorm_sharded(self.out_plan, self.y_bufs, self.ymax if self.fuse_max else None, cfg.groups,
                             cfg.eps, self.gamma, self.beta, self.z_bufs, self.ws, stream)

    def norm_partials(self, stream=None) -> None:
        st_groupnorm_partials(self.out_plan, self.y_bufs, self.ymax if self.fuse_max else None,
                              self.cfg.groups, self.ws, stream)

    def norm_combine(self, stream=None) -> None:
        st_groupnorm_combine(self.out_plan, self.cfg.groups, self.cfg.eps, self.gamma, self.beta, self.ws, stream)

    def norm_apply(self, stream=None) -> None:
        st_groupnorm_apply(self.out_plan, self.y_bufs, self.cfg.groups, self.z_bufs, self.ws, stream)

    def norm_combine_apply(self, stream=None) -> None:
        cfg = self.cfg
        st_groupnorm_combine_apply(self.out_plan, self.y_bufs, cfg.groups, cfg.eps, self.gamma, self.beta,
                                   self.z_bufs, self.ws, stream)

    # ---------------------------------------------------------- backward
    def alloc_backward(self) -> None:
        """Buffers of the GroupNorm backward pass: dz (upstream gradient at
        z), dy (gradient at y), dgamma, dbeta and the backward workspace."""
        torch = _torch()
        cfg = self.cfg
        self.dz_bufs = [torch.zeros_like(y) for y in self.y_bufs]
        self.dy_bufs = [torch.empty_like(y) for y in self.y_bufs]
        self.dgamma = torch.empty(cfg.cout, dtype=torch.float32, device=self.device)
        self.dbeta = torch.empty(cfg.cout, dtype=torch.float32, device=self.device)
        self.bws = torch.zeros(st_groupnorm_backward_workspace_bytes(self.out_plan, cfg.groups),
                               dtype=torch.uint8, device=self.device)

    def load_upstream_grad(self, dz: np.ndarray) -> None:
        """dz: channels-last [N, *spatial, Cout] float32."""
        for i in range(self.S):
            self.out_view(self.dz_bufs, i).copy_(self._host_to_dev(dz[self._global_slices(i)]))
        _torch().cuda.synchronize()

    def norm_backward(self, dzmax=None, dy_bufs=None, stream=None, dy_plan=None) -> None:
        """GroupNorm backward from the forward pass's y and workspace.  With
        dy_plan (e.g. the input-gradient layer's padded input plan) dy goes
        straight into dy_bufs in that plan's layout and dtype."""
        cfg = self.cfg
        st_groupnorm_backward(self.out_plan, self.y_bufs, self.dz_bufs, self.ymax if self.fuse_max else None,
                              dzmax, cfg.groups, self.gamma, self.ws,
                              self.dy_bufs if dy_bufs is None else dy_bufs, self.dgamma, self.dbeta, self.bws,
                              stream, dy_plan=dy_plan)

    def step(self, stream=None) -> None:
        self.exchange(True, stream)
        self.conv(stream)
        self.norm(stream)

    # ----------------------------------------------------------- outputs
    def out_view(self, bufs, i: int):
        return bufs[i].view(self.out_plan.padded_shape(i))

    def gather(self, bufs) -> np.ndarray:
        cfg = self.cfg
        out = np.empty((cfg.batch, *cfg.spatial, cfg.cout), np.float32)
        for i in range(self.S):
            out[self._global_slices(i)] = self.out_view(bufs, i).cpu().numpy()
        return out

    def gather_rows(self, bufs, r0: int, r1: int) -> np.ndarray:
        """Rows [r0, r1) of the outermost spatial axis of an output tensor,
        assembled from the shards that hold them: [N, r1 - r0, *rest, Cout]."""
        cfg = self.cfg
        out = np.empty((cfg.batch, r1 - r0, *cfg.spatial[1:], cfg.cout), np.float32)
        for i in range(self.S):
            inf = self.info[i]
            o0, e0 = inf["offset"][0], inf["extent"][0]
            a, b = max(r0, o0), min(r1, o0 + e0)
            if a >= b:
                continue
            part = self.out_view(bufs, i)[:, a - o0:b - o0].cpu().numpy()
            sl = [slice(None), slice(a - r0, b - r0)] + [slice(o, o + e) for o, e in
                                                         zip(inf["offset"][1:], inf["extent"][1:])]
            out[tuple(sl)] = part
        return out

    def y_host(self) -> np.ndarray:
        return self.gather(self.y_bufs)

    def z_host(self) -> np.ndarray:
        return self.gather(self.z_bufs)

    def at(self, bufs, positions: np.ndarray) -> np.ndarray:
        """Values [P, Cout] at global positions (n, *spatial) (gathered on the GPU)."""
        torch = _torch()
        out = np.empty((len(positions), self.cfg.cout), np.float32)
        pos = np.asarray(positions)
        for i in range(self.S):
            inf = self.info[i]
            lo = np.array(inf["offset"])
            hi = lo + np.array(inf["extent"])
            mask = np.all((pos[:, 1:] >= lo) & (pos[:, 1:] < hi), axis=1)
            if not mask.any():
                continue
            local = pos[mask].copy()
            local[:, 1:] -= lo
            v = self.out_view(bufs, i)
            idx = tuple(torch.from_numpy(local[:, a]).to(self.device) for a in range(local.shape[1]))
            out[mask] = v[idx].cpu().numpy()
        return out

    def gn_state(self) -> dict:
        """Per-shard partial sums, (mean, rstd) and exponents from the workspace."""
        cfg = self.cfg
        lay = st_groupnorm_workspace_layout(self.out_plan, cfg.groups)
        ws = self.ws.cpu().numpy()
        S, N, G = self.S, cfg.batch, cfg.groups
        part = ws[lay["partials_offset"]:lay["partials_offset"] + S * N * G * 16].view(np.float64)
        stats = ws[lay["stats_offset"]:lay["stats_offset"] + N * G * 8].view(np.float32)
        scales = ws[lay["scales_offset"]:lay["scales_offset"] + N * G * 8].view(np.int32)
        return {"partials": part.reshape(S, N, G, 2), "stats": stats.reshape(N, G, 2),
                "scales": scales.reshape(N, G, 2)}

    def padded_host(self, i: int) -> np.ndarray:
        v = self.padded_view(i).cpu().numpy()
        return v.view(np.uint16) if self.dtype == ST_BF16 else v


def dgrad_config(cfg):
    """The layer whose conv is the input gradient of cfg's conv: it reads dy
    (cfg.cout channels, the same shards and halo; exchanged like x) and writes
    dx (cfg.cin channels).  Its GroupNorm part is not used."""
    return dataclasses.replace(cfg, name=f"{cfg.name}_dgrad", cin=cfg.cout, cout=cfg.cin, groups=1)
