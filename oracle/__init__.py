"""CPU oracle for the fused Conv/MatMul -> BatchNorm -> activation operator.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It shares no code
with the HIP library under ``dl_fusion_amd`` and never calls it.

The arithmetic lives in ``oracle.c`` (plain binary64 loops, compiled with gcc
and OpenMP); this module only widens stored inputs to binary64 and composes the
steps in the order the pages define the operator (no BN folding):

  conv (or matmul) -> BatchNorm (or bias add) -> [+ residual] -> activation
  -> [static fp8 quantisation]

Sources (web pages; the section named is where the definition appears):
  [OPPL] "OpenPPL算子融合深度解析：从图优化到推理性能提升" - §3.1 BN inference
         transform and folding, §3.3 residual as an epilogue, §4.3 epilogue
         order bias -> residual -> activation and the GELU(tanh) form.
  [INFR] discosf.com fusion article ("企业官网建设流程全解析") - §2.1 fold
         derivation, §3.3 direct convolution loop.
  [CANN] aitangshan.cn graph-autofusion article - MatMul -> BiasAdd -> act chain.
  [RFC]  MindIE-SD RFC "自动融合..." - §3.4 quantised MatMul + activation.
  [FRT]  "FlashRT 跨层融合深度解析" - §3 static-scale FP8 epilogue.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIBRARY names another build of oracle.c (the sanitizer build); by default the in-tree one
_LIB_PATH = os.environ.get("ORACLE_LIBRARY") or os.path.join(HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    sig = {
        "orc_num_threads": (ctypes.c_int, []),
        "orc_conv2d_nhwc": (None, [_i64] * 11 + [_dp, _dp, _dp, _dp]),
        "orc_conv2d_nhwc_at": (None, [_i64] * 10 + [_dp, _dp, _dp, _i64, _i64p, _dp]),
        "orc_matmul_nt": (None, [_i64, _i64, _i64, _dp, _dp, _dp]),
        "orc_batchnorm": (None, [_i64, _i64, _dp, _dp, _dp, _dp, _dp, ctypes.c_double, _dp]),
        "orc_bias_add": (None, [_i64, _i64, _dp, _dp, _dp]),
        "orc_add": (None, [_i64, _dp, _dp, _dp]),
        "orc_relu": (None, [_i64, _dp, _dp]),
        "orc_gelu_tanh": (None, [_i64, _dp, _dp]),
        "orc_gelu_erf": (None, [_i64, _dp, _dp]),
        "orc_silu": (None, [_i64, _dp, _dp]),
        "orc_round_bf16": (None, [_i64, _dp, _dp]),
        "orc_fold_bn": (None, [_i64, _i64, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_double, _dp, _dp]),
        "orc_e4m3_to_double": (ctypes.c_double, [ctypes.c_int]),
        "orc_e4m3_from_double": (ctypes.c_int, [ctypes.c_double]),
        "orc_e4m3_decode": (None, [_i64, _u8p, _dp]),
        "orc_e4m3_encode": (None, [_i64, _dp, _u8p]),
        "orc_quant_f32": (None, [_i64, _fp, ctypes.c_float, _u8p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def num_threads() -> int:
    return int(_load().orc_num_threads())


def _d(a):
    """Contiguous binary64 view (copy if needed)."""
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, typ=_dp):
    return a.ctypes.data_as(typ) if a is not None else None


# ---------------------------------------------------------------------------
# Exact widening of stored values to binary64
# ---------------------------------------------------------------------------
def from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> binary64 (exact: a bf16 value is the top half of an fp32)."""
    u32 = np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    _load().orc_e4m3_decode(codes.size, _ptr(codes, _u8p), _ptr(out))
    return out


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = _d(v)
    out = np.empty(v.shape, dtype=np.uint8)
    _load().orc_e4m3_encode(v.size, _ptr(v), _ptr(out, _u8p))
    return out


def e4m3_value(code: int) -> float:
    return float(_load().orc_e4m3_to_double(int(code)))


def quant_f32(u32: np.ndarray, inv_scale: float) -> np.ndarray:
    """code = Q(fp32(u * inv_scale)) for fp32 u (the epilogue's static quantisation)."""
    u32 = np.ascontiguousarray(u32, dtype=np.float32)
    out = np.empty(u32.shape, dtype=np.uint8)
    _load().orc_quant_f32(u32.size, _ptr(u32, _fp), ctypes.c_float(np.float32(inv_scale)), _ptr(out, _u8p))
    return out


def widen(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Stored activations -> binary64: 'f32' values, 'bf16' bit patterns or 'fp8' e4m3 codes."""
    if dtype == "f32":
        return _d(arr)
    if dtype == "bf16":
        return from_bf16_bits(arr)
    if dtype == "fp8":
        return e4m3_decode(arr)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# Primitive steps (binary64)
# ---------------------------------------------------------------------------
def conv2d(x, w, bias=None, stride=1, pad=1):
    """x [n,h,w,cin], w [cout,kh,kw,cin] -> y [n,ho,wo,cout]  ([INFR] §3.3 loop, NHWC/OHWI)."""
    x, w = _d(x), _d(w)
    n, h, wd, cin = x.shape
    cout, kh, kw, cin2 = w.shape
    assert cin == cin2
    ho = (h + 2 * pad - kh) // stride + 1
    wo = (wd + 2 * pad - kw) // stride + 1
    y = np.empty((n, ho, wo, cout), dtype=np.float64)
    b = _d(bias) if bias is not None else None
    _load().orc_conv2d_nhwc(n, h, wd, cin, cout, kh, kw, stride, stride, pad, pad,
                            _ptr(x), _ptr(w), _ptr(b), _ptr(y))
    return y


def conv2d_at(x, w, pts, bias=None, stride=1, pad=1):
    """The convolution evaluated only at output pixels pts [npts, 3] = (n, ho, wo) -> [npts, cout]."""
    x, w = _d(x), _d(w)
    n, h, wd, cin = x.shape
    cout, kh, kw, _ = w.shape
    pts = np.ascontiguousarray(pts, dtype=np.int64)
    y = np.empty((pts.shape[0], cout), dtype=np.float64)
    b = _d(bias) if bias is not None else None
    _load().orc_conv2d_nhwc_at(h, wd, cin, cout, kh, kw, stride, stride, pad, pad,
                               _ptr(x), _ptr(w), _ptr(b), pts.shape[0], _ptr(pts, _i64p), _ptr(y))
    return y


def matmul_nt(a, b):
    """y[m][n] = sum_k a[m][k] b[n][k]."""
    a, b = _d(a), _d(b)
    m, k = a.shape
    n, k2 = b.shape
    assert k == k2
    y = np.empty((m, n), dtype=np.float64)
    _load().orc_matmul_nt(m, n, k, _ptr(a), _ptr(b), _ptr(y))
    return y


def batchnorm(y, gamma, beta, mean, var, eps):
    """Inference BN over the last (channel) axis ([OPPL] §3.1)."""
    y = _d(y)
    c = y.shape[-1]
    z = np.empty_like(y)
    g, be, mu, va = _d(gamma), _d(beta), _d(mean), _d(var)
    _load().orc_batchnorm(y.size // c if c else 0, c, _ptr(y), _ptr(g), _ptr(be), _ptr(mu), _ptr(va),
                          float(eps), _ptr(z))
    return z


def bias_add(y, bias):
    y = _d(y)
    c = y.shape[-1]
    z = np.empty_like(y)
    b = _d(bias)
    _load().orc_bias_add(y.size // c if c else 0, c, _ptr(y), _ptr(b), _ptr(z))
    return z


def add(a, b):
    a, b = _d(a), _d(b)
    assert a.shape == b.shape
    out = np.empty_like(a)
    _load().orc_add(a.size, _ptr(a), _ptr(b), _ptr(out))
    return out


def relu(u):
    u = _d(u)
    out = np.empty_like(u)
    _load().orc_relu(u.size, _ptr(u), _ptr(out))
    return out


def gelu_tanh(u):
    u = _d(u)
    out = np.empty_like(u)
    _load().orc_gelu_tanh(u.size, _ptr(u), _ptr(out))
    return out


def round_bf16(v):
    """The nearest bfloat16 value of each binary64 value (ties to even), widened back: the
    storage rounding of a bf16 tensor, taken in one step from binary64."""
    v = _d(v)
    out = np.empty_like(v)
    _load().orc_round_bf16(v.size, _ptr(v), _ptr(out))
    return out


def gelu_erf(u):
    """Exact GELU, u Phi(u) ([RFC] §2.1, §2.4)."""
    u = _d(u)
    out = np.empty_like(u)
    _load().orc_gelu_erf(u.size, _ptr(u), _ptr(out))
    return out


def silu(u):
    """SiLU, u / (1 + e^-u): the gate of SwiGLU ([RFC] §2.2 - §2.4)."""
    u = _d(u)
    out = np.empty_like(u)
    _load().orc_silu(u.size, _ptr(u), _ptr(out))
    return out


def activation(u, act: str):
    if act == "relu":
        return relu(u)
    if act == "gelu_tanh":
        return gelu_tanh(u)
    if act == "gelu_erf":
        return gelu_erf(u)
    if act == "silu":
        return silu(u)
    if act == "none":
        return _d(u)
    raise ValueError(act)


def fold_bn(w, conv_bias, gamma, beta, mean, var, eps):
    """Fold self-check ([OPPL] §3.1, [INFR] §2.1): returns (W', b') in binary64, W' shaped like w."""
    w = _d(w)
    cout = w.shape[0]
    kdim = w.size // cout if cout else 0
    w_out = np.empty_like(w)
    b_out = np.empty(cout, dtype=np.float64)
    cb = _d(conv_bias) if conv_bias is not None else None
    _load().orc_fold_bn(cout, kdim, _ptr(w), _ptr(cb), _ptr(_d(gamma)), _ptr(_d(beta)),
                        _ptr(_d(mean)), _ptr(_d(var)), float(eps), _ptr(w_out), _ptr(b_out))
    return w_out, b_out


# ---------------------------------------------------------------------------
# Whole operator, unfolded ([OPPL] §3.1, §3.3, §4.3 epilogue order)
# ---------------------------------------------------------------------------
def conv_bn_act(inp: dict, pts=None, eps=None):
    """Conv (+conv bias) -> BN -> [+ residual] -> act for a conv workload, in binary64.

    pts: optional [npts, 3] output pixels; then the result is [npts, cout].
    eps: override of the BN epsilon (used by the negative control only).
    """
    wl = inp["workload"]
    x = widen(inp["x"], wl.dtype)
    w = _d(inp["w"])
    eps = inp["eps"] if eps is None else eps
    if pts is None:
        y = conv2d(x, w, inp["conv_bias"], wl.stride, wl.pad)
    else:
        y = conv2d_at(x, w, pts, inp["conv_bias"], wl.stride, wl.pad)
    z = batchnorm(y, inp["gamma"], inp["beta"], inp["mean"], inp["var"], eps)
    if inp.get("residual") is not None:
        r = widen(inp["residual"], wl.dtype)
        if pts is not None:
            p = np.asarray(pts)
            r = r[p[:, 0], p[:, 1], p[:, 2], :]
        z = add(z, r)
    return activation(z, wl.act)


def gemm_bias_act(inp: dict, rows=None):
    """MatMul -> BiasAdd -> act ([CANN] MatMul->BiasAdd->act chain; [RFC] §3.5 Linear + act)."""
    wl = inp["workload"]
    x = widen(inp["x"], "bf16")
    if rows is not None:
        x = x[np.asarray(rows)]
    y = matmul_nt(x, widen(inp["w"], "bf16"))
    if inp.get("bias") is not None:
        y = bias_add(y, inp["bias"])
    return activation(y, wl.act)


def gemm_bias_act_split(inp: dict, parts: int, rows=None):
    """One MatMul over weights concatenated along the output dimension at load, with bias and
    activation, split by columns into `parts` equal tensors ([OPPL] §3.2: the Q, K and V
    projections as one [3 h, h] GEMM whose result is cut into Q, K and V)."""
    y = gemm_bias_act(inp, rows)
    n = y.shape[1]
    if parts < 1 or n % parts:
        raise ValueError("columns must split evenly")
    w = n // parts
    return [np.ascontiguousarray(y[:, p * w:(p + 1) * w]) for p in range(parts)]


def gemm_gated(inp: dict, gate: str, rows=None):
    """Gated projection: one MatMul over gate and up weights interleaved by rows at load (row
    2j = gate j, row 2j+1 = up j), bias added, then out[:, j] = gate_act(g_j) * u_j: SwiGLU
    with gate = "silu", GELU x Mul with "gelu_tanh" / "gelu_erf" ([RFC] §2.2 GMM + SwiGLU,
    §2.3 gated Linear, §2.4 gelu(x) * y).  Returns [m][n/2] in binary64."""
    wl = inp["workload"]
    x = widen(inp["x"], "bf16")
    if rows is not None:
        x = x[np.asarray(rows)]
    y = matmul_nt(x, widen(inp["w"], "bf16"))
    if inp.get("bias") is not None:
        y = bias_add(y, inp["bias"])
    if y.shape[1] % 2:
        raise ValueError("interleaved gate/up needs an even column count")
    return activation(np.ascontiguousarray(y[:, 0::2]), gate) * y[:, 1::2]


def ffn(inp: dict, rows=None):
    """Transformer feed-forward block, FC1 -> activation -> FC2 ([OPPL] §3.2, the FFN fusion:
    two fully connected layers with an activation between them), with the second layer's
    bias and the block's residual add in its epilogue ([OPPL] §3.3):
        y = act(x W1^T + b1) W2^T + b2 [+ residual]
    in binary64 from the stored bf16 tensors.  rows: optional token indices.  Returns
    [rows][d_model]."""
    wl = inp["workload"]
    x = widen(inp["x"], "bf16")
    if rows is not None:
        x = x[np.asarray(rows)]
    h = activation(bias_add(matmul_nt(x, widen(inp["w1"], "bf16")), inp["b1"]), wl.act)
    y = bias_add(matmul_nt(h, widen(inp["w2"], "bf16")), inp["b2"])
    if inp.get("residual") is not None:
        r = widen(inp["residual"], "bf16")
        y = add(y, r if rows is None else r[np.asarray(rows)])
    return y


def fp8_gemm_bn_act_quant(inp: dict, act: str = "relu", rows=None):
    """fp8 MatMul with static scales -> BN -> activation -> static e4m3 quantisation.

    acc = sum_k dec(xq) dec(wq) (exact in binary64); y = acc * s_x * s_w;
    z = BN(y); u = act(z); code = Q(u / s_y).   ([RFC] §3.4, [FRT] §3, [OPPL] §6.4;
    with a GELU, the quantised MatMul + GELU of [RFC] §2.1, whose GELU is tanh or erf)
    Returns (codes uint8, u binary64); u is also the value a bf16 output rounds.
    """
    x = e4m3_decode(inp["x"] if rows is None else inp["x"][np.asarray(rows)])
    w = e4m3_decode(inp["w"])
    acc = matmul_nt(x, w)
    y = acc * inp["s_x"] * inp["s_w"]
    z = batchnorm(y, inp["gamma"], inp["beta"], inp["mean"], inp["var"], inp["eps"])
    u = activation(z, act)
    v = u / inp["s_y"]
    return e4m3_encode(v), u


def fp8_gemm_bn_relu_quant(inp: dict, rows=None):
    """The fp8 pipeline with ReLU (the config of the fp8 workload)."""
    return fp8_gemm_bn_act_quant(inp, "relu", rows)


# ---------------------------------------------------------------------------
# Comparison metric shared by the parity tests
# ---------------------------------------------------------------------------
def rel_error(got, ref, floor_of=None) -> float:
    """max_i |g_i - o_i| / max(|o_i|, rms_c(f)): the relative error, floored at the rms of
    the element's output channel c (the last axis; a 1-D array is one channel) of f = ref, or
    of f = floor_of (same shape) where given: the value before the activation, for a step whose
    activation follows every rounding of the method.

    A plain element-wise relative error is ill-posed where ReLU/GELU outputs are ~0, so
    it is floored.  The floor is per channel because the BN fold multiplies each output
    channel by its own scale gamma/sqrt(var + eps) ("OpenPPL算子融合深度解析" §3.1),
    which can differ by 10x or more between channels (§6.2 of the same page on extreme
    channels): the rounding error of a channel's bf16 weights grows with that channel's
    scale, so it is measured against that channel's magnitude."""
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    if o.size == 0:
        return 0.0
    c = o.shape[-1] if o.ndim > 1 else 1
    g2 = g.reshape(-1, c)
    o2 = o.reshape(-1, c)
    f2 = o2 if floor_of is None else np.asarray(floor_of, dtype=np.float64).reshape(-1, c)
    rms = np.sqrt(np.mean(f2 * f2, axis=0))
    rms = np.where(rms > 0, rms, 1.0)
    den = np.maximum(np.abs(o2), rms[None, :])
    return float(np.max(np.abs(g2 - o2) / den))
