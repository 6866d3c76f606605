"""Layer objects over the C ABI: load-time folding + device buffers + the fused
call and the unfused comparison chain.

A layer is built once from host parameters (fp32 masters, as a model loader
would hold them): BatchNorm is folded on the host by ``dlf_fold_bn`` /
``dlf_bn_scale_shift`` (load time, not per inference), the results are copied
to the GPU once, and ``forward()`` enqueues the single fused kernel.
``forward_unfused()`` runs the separate conv/GEMM, BN (or bias-add), residual
add, activation and quantisation kernels, each through device memory, for the
HBM-traffic and timing comparison.

Where the library has no fused kernel for a layer it says so with
DLF_ERR_UNSUPPORTED, before launching anything; ``forward()`` then runs the
unfused chain in its place, for that call and every later one ("OpenPPL算子融合
深度解析" §4.2 keeps the separate ops where a fusion does not apply; the MindIE-SD
RFC §3.7 falls back to the original graph).  Every other error is raised.

Inputs arrive as host numpy arrays in their storage format (float32 values,
bf16 bit patterns as uint16, or e4m3 codes as uint8).
"""
from __future__ import annotations

import numpy as np
import torch

from . import (DLF_ERR_UNSUPPORTED, DlfError, dlf_act_apply, dlf_add, dlf_bn_apply, dlf_bn_scale_shift,
               dlf_conv_fused, dlf_conv_plain, dlf_ffn_fused_ws, dlf_ffn_pack, dlf_ffn_workspace_bytes, ffn_desc,
               dlf_fold_bn, dlf_gemm_fused, dlf_gemm_plain, dlf_quant_apply, dlf_scale_shift_apply,
               conv_desc, gemm_desc)


def to_device(arr: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Host storage array -> device tensor: 'f32' float32, 'bf16' uint16 bits, 'fp8' uint8 codes."""
    if arr is None:
        return None
    arr = np.ascontiguousarray(arr)
    if dtype == "f32":
        return torch.from_numpy(arr.astype(np.float32, copy=False)).to(device)
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "fp8":
        return torch.from_numpy(arr.view(np.uint8)).to(device)
    raise ValueError(dtype)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor -> host storage array (inverse of to_device)."""
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if dtype == "fp8":
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def _torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[dtype]


class _FallbackLayer:
    """forward() = the fused call, or the unfused chain once the library has answered
    DLF_ERR_UNSUPPORTED for this layer."""

    fused_ok = True

    def forward(self, stream=None, y=None, **kw):
        out = self.y if y is None else y
        if self.fused_ok:
            try:
                self._fused(out, stream, **kw)
                return out
            except DlfError as e:
                if e.status != DLF_ERR_UNSUPPORTED:
                    raise
                self.fused_ok = False
                self.unsupported = e.detail
        return self.forward_unfused(stream, y=out, **kw)


def _master_cast(w: np.ndarray, dtype: str) -> np.ndarray:
    """Unfolded fp32 master weights in the layer's storage type (unfused chain only)."""
    if dtype == "f32":
        return np.ascontiguousarray(w, dtype=np.float32)
    t = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


class FusedConvBNAct(_FallbackLayer):
    """Conv2d (NHWC / OHWI) -> BatchNorm -> [+ residual] -> activation."""

    def __init__(self, inp: dict, device="cuda", with_unfused=True):
        wl = inp["workload"]
        self.wl = wl
        self.dtype = wl.dtype
        self.desc = conv_desc(wl.n, wl.h, wl.w, wl.cin, wl.cout, wl.kh, wl.kw, wl.stride, wl.pad, wl.dtype, wl.act)
        self.desc_plain = conv_desc(wl.n, wl.h, wl.w, wl.cin, wl.cout, wl.kh, wl.kw, wl.stride, wl.pad, wl.dtype,
                                    "none")
        # load time: fold BN into W and b (host, binary64, one rounding)
        w_f, b_f = dlf_fold_bn(inp["w"], inp["conv_bias"], inp["gamma"], inp["beta"], inp["mean"], inp["var"],
                               inp["eps"], wl.dtype)
        self.w_folded_host, self.b_folded_host = w_f, b_f
        self.x = to_device(inp["x"], wl.dtype, device)
        self.w = to_device(w_f, wl.dtype, device)
        self.b = torch.from_numpy(b_f).to(device)
        self.res = to_device(inp.get("residual"), wl.dtype, device)
        self.out_shape = (wl.n, wl.ho, wl.wo, wl.cout)
        self.y = torch.empty(self.out_shape, dtype=_torch_dtype(wl.dtype), device=device)
        self._inp, self._device = inp, device
        self.with_unfused = with_unfused
        if with_unfused:
            self._unfused_buffers()

    def _unfused_buffers(self):
        if getattr(self, "t1", None) is not None:
            return
        inp, wl, device = self._inp, self.wl, self._device
        self.w_raw = to_device(_master_cast(inp["w"], wl.dtype), wl.dtype, device)
        cb = inp["conv_bias"]
        self.conv_bias = torch.from_numpy(np.asarray(cb, np.float32)).to(device) if cb is not None else None
        self.bn = [torch.from_numpy(np.asarray(inp[k], np.float32)).to(device)
                   for k in ("gamma", "beta", "mean", "var")]
        self.eps = inp["eps"]
        self.t1 = torch.empty_like(self.y)
        self.t2 = torch.empty_like(self.y)
        self.y_unfused = torch.empty_like(self.y)

    @property
    def rows(self):
        return self.wl.n * self.wl.ho * self.wl.wo

    def _fused(self, out, stream, x=None, residual=None):
        dlf_conv_fused(self.desc, self.x if x is None else x, self.w, self.b,
                       self.res if residual is None else residual, out, stream)

    def forward_unfused(self, stream=None, y=None, x=None, residual=None):
        wl = self.wl
        self._unfused_buffers()
        out = self.y_unfused if y is None else y
        res = self.res if residual is None else residual
        dlf_conv_plain(self.desc_plain, self.x if x is None else x, self.w_raw, self.conv_bias, self.t1, stream)
        dlf_bn_apply(self.rows, wl.cout, wl.dtype, self.t1, *self.bn, self.eps, self.t2, stream)
        cur = self.t2
        if res is not None:
            dlf_add(self.t2.numel(), wl.dtype, self.t2, res, self.t1, stream)
            cur = self.t1
        dlf_act_apply(cur.numel(), wl.dtype, wl.act, cur, out, stream)
        return out


class FusedLinearAct(_FallbackLayer):
    """MatMul (x W^T, W in [out][in]) -> + bias -> activation, bf16 in/out."""

    def __init__(self, inp: dict, device="cuda", with_unfused=True):
        wl = inp["workload"]
        self.wl = wl
        self.desc = gemm_desc(wl.m, wl.n, wl.k, "bf16", "bf16", wl.act)
        self.desc_plain = gemm_desc(wl.m, wl.n, wl.k, "bf16", "bf16", "none")
        self.x = to_device(inp["x"], "bf16", device)
        self.w = to_device(inp["w"], "bf16", device)
        self.bias = torch.from_numpy(inp["bias"]).to(device) if inp.get("bias") is not None else None
        self.y = torch.empty((wl.m, wl.n), dtype=torch.bfloat16, device=device)
        self.with_unfused = with_unfused
        if with_unfused:
            self._unfused_buffers()

    def _unfused_buffers(self):
        if getattr(self, "t1", None) is None:
            self.t1 = torch.empty_like(self.y)
            self.t2 = torch.empty_like(self.y)
            self.y_unfused = torch.empty_like(self.y)

    def _fused(self, out, stream, residual=None):
        dlf_gemm_fused(self.desc, self.x, self.w, None, self.bias, residual, out, stream)

    def forward_unfused(self, stream=None, y=None, residual=None):
        wl = self.wl
        self._unfused_buffers()
        out = self.y_unfused if y is None else y
        dlf_gemm_plain(self.desc_plain, self.x, self.w, 1.0, self.t1, stream)
        cur, free = self.t1, self.t2
        if self.bias is not None:
            dlf_scale_shift_apply(wl.m, wl.n, "bf16", cur, None, self.bias, free, stream)
            cur, free = free, cur
        if residual is not None:
            dlf_add(cur.numel(), "bf16", cur, residual, free, stream)
            cur, free = free, cur
        dlf_act_apply(cur.numel(), "bf16", wl.act, cur, out, stream)
        return out


class Fp8LinearBNReluQuant(_FallbackLayer):
    """fp8 e4m3 MatMul with static scales -> folded BN scale/shift -> ReLU -> static e4m3 output."""

    def __init__(self, inp: dict, device="cuda", with_unfused=True):
        wl = inp["workload"]
        self.wl = wl
        self.s_x, self.s_w, self.s_y = inp["s_x"], inp["s_w"], inp["s_y"]
        self.inv_s_y = float(np.float32(1.0 / self.s_y))
        # load time: BN as a per-channel (alpha, beta') epilogue, alpha absorbing s_x * s_w
        alpha, shift = dlf_bn_scale_shift(inp["conv_bias"], inp["gamma"], inp["beta"], inp["mean"], inp["var"],
                                          inp["eps"], float(self.s_x) * float(self.s_w))
        self.alpha_host, self.shift_host = alpha, shift
        self.desc = gemm_desc(wl.m, wl.n, wl.k, "fp8", "fp8", "relu", self.inv_s_y)
        self.desc_plain = gemm_desc(wl.m, wl.n, wl.k, "fp8", "f32", "none")
        self.x = to_device(inp["x"], "fp8", device)
        self.w = to_device(inp["w"], "fp8", device)
        self.alpha = torch.from_numpy(alpha).to(device)
        self.shift = torch.from_numpy(shift).to(device)
        self.y = torch.empty((wl.m, wl.n), dtype=torch.uint8, device=device)
        self._inp, self._device = inp, device
        self.with_unfused = with_unfused
        if with_unfused:
            self._unfused_buffers()

    def _unfused_buffers(self):
        if getattr(self, "t1", None) is not None:
            return
        inp, wl, device = self._inp, self.wl, self._device
        self.bn = [torch.from_numpy(np.asarray(inp[k], np.float32)).to(device)
                   for k in ("gamma", "beta", "mean", "var")]
        self.eps = inp["eps"]
        self.dequant = float(np.float32(float(self.s_x) * float(self.s_w)))
        self.t1 = torch.empty((wl.m, wl.n), dtype=torch.float32, device=device)
        self.t2 = torch.empty_like(self.t1)
        self.y_unfused = torch.empty_like(self.y)

    def _fused(self, out, stream):
        dlf_gemm_fused(self.desc, self.x, self.w, self.alpha, self.shift, None, out, stream)

    def forward_unfused(self, stream=None, y=None):
        wl = self.wl
        self._unfused_buffers()
        out = self.y_unfused if y is None else y
        dlf_gemm_plain(self.desc_plain, self.x, self.w, self.dequant, self.t1, stream)
        dlf_bn_apply(wl.m, wl.n, "f32", self.t1, *self.bn, self.eps, self.t2, stream)
        dlf_act_apply(self.t2.numel(), "f32", "relu", self.t2, self.t2, stream)
        dlf_quant_apply(self.t2.numel(), self.t2, self.inv_s_y, out, stream)
        return out


class FusedFFN(_FallbackLayer):
    """Transformer feed-forward block: dlf_ffn_fused_ws (weights packed once at load by
    dlf_ffn_pack, and the workspace its d_ff split asks for, allocated at load); the unfused
    form is FC1 (+ b1, act) and FC2 (+ b2, + residual) as two GEMMs with their own register
    epilogues, the intermediate going through HBM.  A block the fused kernel is not built for
    (d_model outside 256/512/768/1024, d_ff not a multiple of 256) runs the two GEMMs."""

    def __init__(self, inp: dict, device="cuda", with_unfused=True):
        wl = inp["workload"]
        self.wl = wl
        self.desc = ffn_desc(wl.m, wl.d_model, wl.d_ff, wl.act)
        self.x = to_device(inp["x"], "bf16", device)
        self.b1 = torch.from_numpy(inp["b1"]).to(device)
        self.b2 = torch.from_numpy(inp["b2"]).to(device)
        self.res = to_device(inp.get("residual"), "bf16", device)
        self.y = torch.empty((wl.m, wl.d_model), dtype=torch.bfloat16, device=device)
        self._inp, self._device = inp, device
        try:
            self.ws_bytes = dlf_ffn_workspace_bytes(self.desc)
        except DlfError as e:
            if e.status != DLF_ERR_UNSUPPORTED:
                raise
            self.fused_ok, self.unsupported, self.ws_bytes = False, e.detail, 0
        if self.fused_ok:
            self.w1p = to_device(dlf_ffn_pack(inp["w1"]), "bf16", device)
            self.w2p = to_device(dlf_ffn_pack(inp["w2"]), "bf16", device)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device) if self.ws_bytes else None
        self.with_unfused = with_unfused
        if with_unfused or not self.fused_ok:
            self._unfused_buffers()

    def _unfused_buffers(self):
        if getattr(self, "h", None) is not None:
            return
        inp, wl, device = self._inp, self.wl, self._device
        self.w1 = to_device(inp["w1"], "bf16", device)
        self.w2 = to_device(inp["w2"], "bf16", device)
        self.desc1 = gemm_desc(wl.m, wl.d_ff, wl.d_model, "bf16", "bf16", wl.act)
        self.desc2 = gemm_desc(wl.m, wl.d_model, wl.d_ff, "bf16", "bf16", "none")
        self.h = torch.empty((wl.m, wl.d_ff), dtype=torch.bfloat16, device=device)
        self.y_unfused = torch.empty_like(self.y)

    def _fused(self, out, stream):
        dlf_ffn_fused_ws(self.desc, self.x, self.w1p, self.b1, self.w2p, self.b2, self.res, out, self.ws,
                         self.ws_bytes, stream)

    def forward_unfused(self, stream=None, y=None):
        self._unfused_buffers()
        out = self.y_unfused if y is None else y
        dlf_gemm_fused(self.desc1, self.x, self.w1, None, self.b1, None, self.h, stream)
        dlf_gemm_fused(self.desc2, self.h, self.w2, None, self.b2, self.res, out, stream)
        return out


def make_layer(inp: dict, device="cuda", with_unfused=True):
    kind = inp["workload"].kind
    if kind == "conv":
        return FusedConvBNAct(inp, device, with_unfused)
    if kind == "gemm":
        return FusedLinearAct(inp, device, with_unfused)
    if kind == "ffn":
        return FusedFFN(inp, device, with_unfused)
    return Fp8LinearBNReluQuant(inp, device, with_unfused)
