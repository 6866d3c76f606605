"""Python binding of libdlfusion, the fused Conv/MatMul -> BatchNorm -> activation
operator for MI355X (gfx950).

This module only marshals arguments to the C ABI declared in
``include/dlfusion.h`` (same function names).  Every step of the operator runs
in the library's HIP kernels or its host fold; there is no Python or CPU
fallback: importing fails loudly when ``libdlfusion.so`` has not been built.

Device buffers are passed as contiguous torch tensors (their ``data_ptr()``)
or as raw integer addresses; host buffers of the fold functions are numpy
arrays.  ``stream=None`` means torch's current stream on the current device.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# DLF_LIBRARY names another build of the same library (the sanitizer build of the host code the
# CPU test-suite runs under); by default the in-tree build
LIB_PATH = os.environ.get("DLF_LIBRARY") or os.path.join(_HERE, "libdlfusion.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first (python -c 'import __graft_entry__ as g; g.build()')")

# torch's ROCm build carries its own HIP runtime under the same soname as the system one the
# library links against.  Loading torch first makes the library bind to that runtime, so one
# HIP runtime serves the process; with the library loaded first, its calls found no device
# while torch's allocations went on working.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

# ---------------------------------------------------------------------------
# Enums and descriptors (mirror include/dlfusion.h)
# ---------------------------------------------------------------------------
DLF_OK, DLF_ERR_INVALID_ARG, DLF_ERR_UNSUPPORTED, DLF_ERR_HIP, DLF_ERR_ALIAS = 0, -1, -2, -3, -4
DLF_F32, DLF_BF16, DLF_FP8_E4M3 = 0, 1, 2
DLF_ACT_NONE, DLF_ACT_RELU, DLF_ACT_GELU_TANH, DLF_ACT_GELU_ERF = 0, 1, 2, 3

DTYPES = {"f32": DLF_F32, "bf16": DLF_BF16, "fp8": DLF_FP8_E4M3}
ACTS = {"none": DLF_ACT_NONE, "relu": DLF_ACT_RELU, "gelu_tanh": DLF_ACT_GELU_TANH, "gelu_erf": DLF_ACT_GELU_ERF}
DLF_GATE_SILU, DLF_GATE_GELU_TANH, DLF_GATE_GELU_ERF = 0, 1, 2
GATES = {"silu": DLF_GATE_SILU, "gelu_tanh": DLF_GATE_GELU_TANH, "gelu_erf": DLF_GATE_GELU_ERF}


class dlf_conv_desc(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("h", ctypes.c_int64), ("w", ctypes.c_int64),
                ("c_in", ctypes.c_int64), ("c_out", ctypes.c_int64), ("kh", ctypes.c_int64),
                ("kw", ctypes.c_int64), ("stride_h", ctypes.c_int32), ("stride_w", ctypes.c_int32),
                ("pad_h", ctypes.c_int32), ("pad_w", ctypes.c_int32), ("dtype", ctypes.c_int),
                ("act", ctypes.c_int)]


class dlf_gemm_desc(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int), ("act", ctypes.c_int),
                ("out_inv_scale", ctypes.c_float)]


def conv_desc(n, h, w, c_in, c_out, kh=3, kw=3, stride=1, pad=1, dtype="bf16", act="relu"):
    return dlf_conv_desc(n, h, w, c_in, c_out, kh, kw, stride, stride, pad, pad,
                         DTYPES.get(dtype, dtype), ACTS.get(act, act))


def gemm_desc(m, n, k, in_dtype="bf16", out_dtype="bf16", act="none", out_inv_scale=1.0):
    return dlf_gemm_desc(m, n, k, DTYPES.get(in_dtype, in_dtype), DTYPES.get(out_dtype, out_dtype),
                         ACTS.get(act, act), out_inv_scale)


OPS = {"input": 0, "conv": 1, "matmul": 2, "matmul_fp8": 3, "bias_add": 4, "batchnorm": 5, "add": 6,
       "relu": 7, "gelu": 8, "gelu_erf": 9, "quant": 10}
DLF_OP_OTHER = 11
DLF_NODE_OUTPUT, DLF_NODE_TRAINING = 1, 2


class dlf_ffn_desc(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("d_model", ctypes.c_int64), ("d_ff", ctypes.c_int64),
                ("dtype", ctypes.c_int), ("act", ctypes.c_int)]


def ffn_desc(m, d_model, d_ff, act="gelu_tanh", dtype="bf16"):
    return dlf_ffn_desc(m, d_model, d_ff, DTYPES.get(dtype, dtype), ACTS.get(act, act))


class dlf_graph_node(ctypes.Structure):
    _fields_ = [("op", ctypes.c_int32), ("n_inputs", ctypes.c_int32), ("inputs", ctypes.c_int32 * 2),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32), ("rank", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("shape", ctypes.c_int64 * 4), ("flops", ctypes.c_int64)]


class dlf_fusion_group(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int32), ("nodes", ctypes.c_int32 * 5), ("saved_bytes", ctypes.c_int64),
                ("net_benefit", ctypes.c_double)]


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_f32p = ctypes.POINTER(ctypes.c_float)
_SIGS = {
    "dlf_fold_bn": [_i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_double, ctypes.c_int, _vp, _vp],
    "dlf_bn_scale_shift": [_i64, _vp, _vp, _vp, _vp, _vp, ctypes.c_double, ctypes.c_double, _vp, _vp],
    "dlf_conv_fused": [ctypes.POINTER(dlf_conv_desc), _vp, _vp, _vp, _vp, _vp, _vp],
    "dlf_gemm_fused": [ctypes.POINTER(dlf_gemm_desc), _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "dlf_gemm_fused_split": [ctypes.POINTER(dlf_gemm_desc), _vp, _vp, _vp, _vp, ctypes.c_int32,
                             ctypes.POINTER(_vp), _vp],
    "dlf_gemm_fused_gated": [ctypes.POINTER(dlf_gemm_desc), _vp, _vp, _vp, _vp, ctypes.c_int, _vp, _vp],
    "dlf_conv_plain": [ctypes.POINTER(dlf_conv_desc), _vp, _vp, _vp, _vp, _vp],
    "dlf_gemm_plain": [ctypes.POINTER(dlf_gemm_desc), _vp, _vp, ctypes.c_float, _vp, _vp],
    "dlf_bn_apply": [_i64, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, ctypes.c_double, _vp, _vp],
    "dlf_scale_shift_apply": [_i64, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _vp],
    "dlf_add": [_i64, ctypes.c_int, _vp, _vp, _vp, _vp],
    "dlf_act_apply": [_i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp],
    "dlf_quant_apply": [_i64, _vp, ctypes.c_float, _vp, _vp],
    "dlf_ffn_pack": [_i64, _i64, _vp, _vp],
    "dlf_ffn_fused": [ctypes.POINTER(dlf_ffn_desc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "dlf_ffn_workspace_bytes": [ctypes.POINTER(dlf_ffn_desc), ctypes.POINTER(ctypes.c_size_t)],
    "dlf_ffn_fused_ws": [ctypes.POINTER(dlf_ffn_desc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                         _vp],
    "dlf_ffn_fused_noalloc": [ctypes.POINTER(dlf_ffn_desc), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "dlf_clock_probe": [ctypes.c_int32, ctypes.c_int32, _vp, _vp],
    "dlf_fusion_plan": [ctypes.POINTER(dlf_graph_node), ctypes.c_int32, ctypes.c_double, ctypes.c_double,
                        ctypes.POINTER(dlf_fusion_group), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)],
}
for _name, _args in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = ctypes.c_int
    _fn.argtypes = _args
_lib.dlf_status_string.restype = ctypes.c_char_p
_lib.dlf_status_string.argtypes = [ctypes.c_int]
_lib.dlf_last_error.restype = ctypes.c_char_p
_lib.dlf_last_error.argtypes = []
_lib.dlf_tuning_reload.restype = None
_lib.dlf_tuning_reload.argtypes = []


class DlfError(RuntimeError):
    def __init__(self, status: int, func: str):
        self.status = status
        self.detail = dlf_last_error()
        super().__init__(f"{func}: {dlf_status_string(status)}: {self.detail}")


def dlf_status_string(status: int) -> str:
    return _lib.dlf_status_string(int(status)).decode()


def dlf_last_error() -> str:
    return _lib.dlf_last_error().decode()


def dlf_tuning_reload():
    """Re-read the DLF_* tuning switches from the environment (the library reads them once,
    when it is loaded)."""
    _lib.dlf_tuning_reload()


def _check(status: int, func: str):
    if status != DLF_OK:
        raise DlfError(status, func)


def _dev(t):
    """Device pointer of a contiguous torch tensor, a raw int address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("device tensors must be contiguous")
    return t.data_ptr()


def _host(a, dtype=None):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(a, dtype=dtype) if dtype is not None else np.ascontiguousarray(a)
    return arr, arr.ctypes.data


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# Host-side fold
# ---------------------------------------------------------------------------
def dlf_fold_bn(w, conv_bias, gamma, beta, mean, var, eps, w_out_dtype="bf16"):
    """Fold BN into conv weights (host, binary64, one RNE rounding).  w is fp32
    [cout, ...] (OHWI); returns (w_out [same shape] as float32 or uint16 bf16 bits,
    bias_out float32 [cout])."""
    w_arr, w_p = _host(w, np.float32)
    cout = w_arr.shape[0] if w_arr.ndim else 0
    k = w_arr.size // cout if cout else 0
    dt = DTYPES.get(w_out_dtype, w_out_dtype)
    out = np.empty(w_arr.shape, dtype=np.float32 if dt == DLF_F32 else np.uint16)
    bias_out = np.empty(cout, dtype=np.float32)
    keep = [_host(v, np.float32) for v in (conv_bias, gamma, beta, mean, var)]
    st = _lib.dlf_fold_bn(cout, k, w_p, *[p for _, p in keep], float(eps), dt, out.ctypes.data,
                          bias_out.ctypes.data)
    _check(st, "dlf_fold_bn")
    return out, bias_out


def dlf_bn_scale_shift(conv_bias, gamma, beta, mean, var, eps, pre_scale=1.0):
    """Per-channel (alpha, beta') with BN(acc * pre_scale + b) = acc * alpha + beta' (host)."""
    g, _ = _host(gamma, np.float32)
    cout = g.size
    scale = np.empty(cout, dtype=np.float32)
    shift = np.empty(cout, dtype=np.float32)
    keep = [_host(v, np.float32) for v in (conv_bias, gamma, beta, mean, var)]
    st = _lib.dlf_bn_scale_shift(cout, *[p for _, p in keep], float(eps), float(pre_scale),
                                 scale.ctypes.data, shift.ctypes.data)
    _check(st, "dlf_bn_scale_shift")
    return scale, shift


# ---------------------------------------------------------------------------
# Device entry points (asynchronous on `stream`)
# ---------------------------------------------------------------------------
def dlf_conv_fused(desc, x, w, bias, residual, y, stream=None):
    _check(_lib.dlf_conv_fused(ctypes.byref(desc), _dev(x), _dev(w), _dev(bias), _dev(residual), _dev(y),
                               _stream(stream)), "dlf_conv_fused")


def dlf_gemm_fused(desc, a, b, col_scale, col_shift, residual, c, stream=None):
    _check(_lib.dlf_gemm_fused(ctypes.byref(desc), _dev(a), _dev(b), _dev(col_scale), _dev(col_shift),
                               _dev(residual), _dev(c), _stream(stream)), "dlf_gemm_fused")


def dlf_gemm_fused_gated(desc, a, b, col_scale, col_shift, gate, c, stream=None):
    """Gated projection: c[:, j] = gate(g_j) * u_j over interleaved (gate, up) weight rows."""
    _check(_lib.dlf_gemm_fused_gated(ctypes.byref(desc), _dev(a), _dev(b), _dev(col_scale), _dev(col_shift),
                                     GATES.get(gate, gate), _dev(c), _stream(stream)), "dlf_gemm_fused_gated")


def dlf_gemm_fused_split(desc, a, b, col_scale, col_shift, outs, stream=None):
    """One GEMM, its columns stored to len(outs) tensors (see include/dlfusion.h)."""
    arr = (_vp * max(1, len(outs)))(*[_dev(o) for o in outs])
    _check(_lib.dlf_gemm_fused_split(ctypes.byref(desc), _dev(a), _dev(b), _dev(col_scale), _dev(col_shift),
                                     len(outs), arr, _stream(stream)), "dlf_gemm_fused_split")


def dlf_conv_plain(desc, x, w, conv_bias, y, stream=None):
    _check(_lib.dlf_conv_plain(ctypes.byref(desc), _dev(x), _dev(w), _dev(conv_bias), _dev(y), _stream(stream)),
           "dlf_conv_plain")


def dlf_gemm_plain(desc, a, b, dequant, y, stream=None):
    _check(_lib.dlf_gemm_plain(ctypes.byref(desc), _dev(a), _dev(b), float(dequant), _dev(y), _stream(stream)),
           "dlf_gemm_plain")


def dlf_bn_apply(rows, c, dt, y, gamma, beta, mean, var, eps, z, stream=None):
    _check(_lib.dlf_bn_apply(rows, c, DTYPES.get(dt, dt), _dev(y), _dev(gamma), _dev(beta), _dev(mean), _dev(var),
                             float(eps), _dev(z), _stream(stream)), "dlf_bn_apply")


def dlf_scale_shift_apply(rows, c, dt, y, scale, shift, z, stream=None):
    _check(_lib.dlf_scale_shift_apply(rows, c, DTYPES.get(dt, dt), _dev(y), _dev(scale), _dev(shift), _dev(z),
                                      _stream(stream)), "dlf_scale_shift_apply")


def dlf_add(count, dt, a, b, out, stream=None):
    _check(_lib.dlf_add(count, DTYPES.get(dt, dt), _dev(a), _dev(b), _dev(out), _stream(stream)), "dlf_add")


def dlf_act_apply(count, dt, act, x, out, stream=None):
    _check(_lib.dlf_act_apply(count, DTYPES.get(dt, dt), ACTS.get(act, act), _dev(x), _dev(out),
                              _stream(stream)), "dlf_act_apply")


def dlf_quant_apply(count, x, inv_scale, codes, stream=None):
    _check(_lib.dlf_quant_apply(count, _dev(x), float(inv_scale), _dev(codes), _stream(stream)),
           "dlf_quant_apply")


def dlf_ffn_pack(w_bits):
    """Host: a [rows][k] bf16 weight (uint16 bit patterns) packed in the fused FFN kernel's
    fragment order; returns a new uint16 array of the same shape."""
    w, _ = _host(w_bits, np.uint16)
    out = np.empty_like(w)
    rows, k = w.shape
    _check(_lib.dlf_ffn_pack(rows, k, w.ctypes.data, out.ctypes.data), "dlf_ffn_pack")
    return out


def dlf_ffn_fused(desc, x, w1_packed, b1, w2_packed, b2, residual, y, stream=None):
    _check(_lib.dlf_ffn_fused(ctypes.byref(desc), _dev(x), _dev(w1_packed), _dev(b1), _dev(w2_packed), _dev(b2),
                              _dev(residual), _dev(y), _stream(stream)), "dlf_ffn_fused")


def dlf_ffn_workspace_bytes(desc):
    n = ctypes.c_size_t(0)
    _check(_lib.dlf_ffn_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "dlf_ffn_workspace_bytes")
    return n.value


def dlf_ffn_fused_ws(desc, x, w1_packed, b1, w2_packed, b2, residual, y, workspace, workspace_bytes, stream=None):
    _check(_lib.dlf_ffn_fused_ws(ctypes.byref(desc), _dev(x), _dev(w1_packed), _dev(b1), _dev(w2_packed), _dev(b2),
                                 _dev(residual), _dev(y), _dev(workspace), int(workspace_bytes), _stream(stream)),
           "dlf_ffn_fused_ws")


DLF_FFN_NOALLOC_SCRATCH_BYTES = 32 << 20


def dlf_ffn_fused_noalloc(desc, x, w1_packed, b1, w2_packed, b2, residual, y, stream=None):
    """dlf_ffn_fused_ws without a workspace: the split's partial sums use the library's static
    device scratch (see include/dlfusion.h)."""
    _check(_lib.dlf_ffn_fused_noalloc(ctypes.byref(desc), _dev(x), _dev(w1_packed), _dev(b1), _dev(w2_packed),
                                      _dev(b2), _dev(residual), _dev(y), _stream(stream)), "dlf_ffn_fused_noalloc")


def dlf_clock_probe(workgroups, iters, stamps, stream=None):
    """Enqueue the shader-clock probe; stamps: a device int64 tensor of 4 * workgroups values."""
    _check(_lib.dlf_clock_probe(int(workgroups), int(iters), _dev(stamps), _stream(stream)), "dlf_clock_probe")


def graph_nodes(graph):
    """A graph given as node dicts (op, inputs, shape, dtype, flops, output, training; op names
    as in OPS, any other name is DLF_OP_OTHER) as a dlf_graph_node array."""
    arr = (dlf_graph_node * len(graph))()
    for i, nd in enumerate(graph):
        x = arr[i]
        x.op = OPS.get(nd["op"], DLF_OP_OTHER)
        ins = list(nd["inputs"])
        if len(ins) > 2:
            raise ValueError(f"node {i}: at most two inputs")
        x.n_inputs = len(ins)
        for j, v in enumerate(ins):
            x.inputs[j] = v
        x.dtype = DTYPES.get(nd["dtype"], nd["dtype"])
        x.flags = (DLF_NODE_OUTPUT if nd.get("output") else 0) | (DLF_NODE_TRAINING if nd.get("training") else 0)
        shp = tuple(nd["shape"])
        if len(shp) > 4:
            raise ValueError(f"node {i}: rank above 4")
        x.rank = len(shp)
        for d, v in enumerate(shp):
            x.shape[d] = v
        x.flops = int(nd.get("flops", 0))
    return arr


def dlf_fusion_plan(graph, ridge, overhead_frac):
    """Groups chosen by the library's fusion pass: a list of dicts with "nodes" (chain order),
    "saved" (bytes) and "net" (bytes), in order of their first node."""
    arr = graph_nodes(graph)
    count = ctypes.c_int32(0)
    cap = max(1, len(graph))        # groups are disjoint and hold two or more nodes each
    out = (dlf_fusion_group * cap)()
    _check(_lib.dlf_fusion_plan(arr, len(graph), float(ridge), float(overhead_frac), out, cap,
                                ctypes.byref(count)), "dlf_fusion_plan")
    return [{"nodes": list(out[i].nodes[:out[i].count]), "saved": int(out[i].saved_bytes),
             "net": float(out[i].net_benefit)} for i in range(count.value)]


def raw():
    """The ctypes library handle (for status-code tests that bypass the raising wrappers)."""
    return _lib
