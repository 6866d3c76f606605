"""CPU tests of libdlfusion's host side: exported symbols, the BN fold and the
argument validation.  No test here launches a kernel: every device call made
below must be rejected (or be a zero-size no-op) before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dlfusion.h")

dlf = pytest.importorskip("dl_fusion_amd", reason="libdlfusion.so not built")


def _gpu_reachable() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# Tests that hand the library fake device addresses run only where no GPU can be
# reached, so that even a validation bug could not launch a kernel on them.
fake_pointers = pytest.mark.skipif(_gpu_reachable(), reason="uses fake device addresses; CPU-only")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dlf_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 13
    lib = ctypes.CDLL(dlf.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert dlf.dlf_status_string(0) == "DLF_OK"
    assert dlf.dlf_status_string(-2) == "DLF_ERR_UNSUPPORTED"
    assert dlf.dlf_status_string(-4) == "DLF_ERR_ALIAS"
    assert dlf.dlf_status_string(7) == "DLF_STATUS_UNKNOWN"


# ---------------------------------------------------------------------------
# BN fold against the oracle's binary64 fold
# ---------------------------------------------------------------------------
def _bf16_to_f64(bits):
    return oracle.from_bf16_bits(bits)


def _assert_correctly_rounded_bf16(bits, exact):
    """bits must be the bf16 nearest to `exact` (no neighbour is strictly closer)."""
    v = _bf16_to_f64(bits)
    up = _bf16_to_f64((bits.astype(np.uint32) + 1).astype(np.uint16))
    dn = _bf16_to_f64((bits.astype(np.uint32) - 1).astype(np.uint16))
    err = np.abs(v - exact)
    assert np.all(err <= np.abs(up - exact)) and np.all(err <= np.abs(dn - exact))


@pytest.mark.parametrize("cfg", [0, 1, 2])
def test_fold_fp32_and_bf16_are_single_roundings_of_the_binary64_fold(cfg):
    wl = workloads.workload(cfg) if cfg == 0 else workloads.workload(cfg, n=1, h=4, w=4)
    inp = workloads.generate(wl)
    ref_w, ref_b = oracle.fold_bn(inp["w"], inp["conv_bias"], inp["gamma"], inp["beta"], inp["mean"],
                                  inp["var"], inp["eps"])
    w32, b32 = dlf.dlf_fold_bn(inp["w"], inp["conv_bias"], inp["gamma"], inp["beta"], inp["mean"], inp["var"],
                               inp["eps"], "f32")
    np.testing.assert_array_equal(w32, ref_w.astype(np.float32))
    np.testing.assert_array_equal(b32, ref_b.astype(np.float32))
    wb, bb = dlf.dlf_fold_bn(inp["w"], inp["conv_bias"], inp["gamma"], inp["beta"], inp["mean"], inp["var"],
                             inp["eps"], "bf16")
    assert wb.dtype == np.uint16 and wb.shape == inp["w"].shape
    _assert_correctly_rounded_bf16(wb.ravel(), ref_w.ravel())
    np.testing.assert_array_equal(bb, b32)


def test_fold_bf16_avoids_double_rounding():
    """W' = w * s lands just above the bf16 midpoint 1 + 2^-8 by less than half an fp32
    ulp: a fold through fp32 would land on the midpoint and tie to even (1.0, 0x3F80);
    the single binary64 -> bf16 rounding must give 1 + 2^-7 (0x3F81)."""
    w = np.array([[1.0 + 2.0 ** -8]], dtype=np.float32)
    eps = 0.25 - 2.0 ** -28                  # var + eps = 1 - 2^-28, so s = 1 + 2^-29 + ...
    s = 1.0 / np.sqrt(0.75 + eps)
    prod = float(w[0, 0]) * s
    assert prod > 1.0 + 2.0 ** -8 and float(np.float32(prod)) == 1.0 + 2.0 ** -8
    wb, _ = dlf.dlf_fold_bn(w, None, np.ones(1), np.zeros(1), np.zeros(1), np.array([0.75], np.float32),
                            eps, "bf16")
    assert wb[0, 0] == 0x3F81


def test_fold_without_bias_synthesises_one():
    inp = workloads.generate(workloads.workload(1, n=1, h=4, w=4))
    _, b_none = dlf.dlf_fold_bn(inp["w"], None, inp["gamma"], inp["beta"], inp["mean"], inp["var"], 1e-5, "f32")
    _, b_zero = dlf.dlf_fold_bn(inp["w"], np.zeros(64, np.float32), inp["gamma"], inp["beta"], inp["mean"],
                                inp["var"], 1e-5, "f32")
    np.testing.assert_array_equal(b_none, b_zero)
    assert np.any(b_none != 0)


def test_fold_uses_eps_exactly():
    inp = workloads.generate(workloads.workload(2, n=1, h=4, w=4))
    st = inp["stressed"]
    w_a, _ = dlf.dlf_fold_bn(inp["w"], None, inp["gamma"], inp["beta"], inp["mean"], inp["var"], 1e-2, "f32")
    ref, _ = oracle.fold_bn(inp["w"], None, inp["gamma"], inp["beta"], inp["mean"], inp["var"], 1e-2)
    np.testing.assert_array_equal(w_a, ref.astype(np.float32))
    w_0, _ = dlf.dlf_fold_bn(inp["w"], None, inp["gamma"], inp["beta"], inp["mean"], inp["var"], 0.0, "f32")
    ratio = np.abs(w_0[st]).max(axis=(1, 2, 3)) / np.abs(w_a[st]).max(axis=(1, 2, 3))
    assert ratio.min() > 3.0


def test_bn_scale_shift_matches_oracle():
    inp = workloads.generate(workloads.workload(4, m=8, n=64, k=32))
    pre = float(inp["s_x"]) * float(inp["s_w"])
    alpha, shift = dlf.dlf_bn_scale_shift(None, inp["gamma"], inp["beta"], inp["mean"], inp["var"], inp["eps"], pre)
    s_ref, b_ref = oracle.fold_bn(np.ones((64, 1)), None, inp["gamma"], inp["beta"], inp["mean"], inp["var"],
                                  inp["eps"])
    exact_alpha = s_ref[:, 0] * pre
    assert np.all(np.abs(alpha - exact_alpha) <= np.spacing(np.abs(alpha).astype(np.float32)) * 1.0 + 0)
    np.testing.assert_array_equal(shift, b_ref.astype(np.float32))
    bias = np.linspace(-1, 1, 64).astype(np.float32)
    _, shift_b = dlf.dlf_bn_scale_shift(bias, inp["gamma"], inp["beta"], inp["mean"], inp["var"], inp["eps"], pre)
    _, b_ref2 = oracle.fold_bn(np.ones((64, 1)), bias, inp["gamma"], inp["beta"], inp["mean"], inp["var"], inp["eps"])
    np.testing.assert_array_equal(shift_b, b_ref2.astype(np.float32))


# ---------------------------------------------------------------------------
# Validation: each failure path returns its status before any HIP call
# ---------------------------------------------------------------------------
def test_fold_rejects_bad_arguments():
    one = np.ones(1, np.float32)
    w = np.ones((1, 9), np.float32)
    for eps in (-1e-5, float("nan"), float("inf")):
        with pytest.raises(dlf.DlfError) as e:
            dlf.dlf_fold_bn(w, None, one, one, one, one, eps, "f32")
        assert e.value.status == dlf.DLF_ERR_INVALID_ARG
    with pytest.raises(dlf.DlfError) as e:
        dlf.dlf_fold_bn(w, None, one, one, one, np.zeros(1, np.float32), 0.0, "f32")   # var + eps == 0
    assert e.value.status == dlf.DLF_ERR_INVALID_ARG and "var + eps" in e.value.detail
    with pytest.raises(dlf.DlfError) as e:
        dlf.dlf_fold_bn(w, None, one, one, one, one, 1e-5, "fp8")
    assert e.value.status == dlf.DLF_ERR_UNSUPPORTED
    lib = dlf.raw()
    assert lib.dlf_fold_bn(1, 9, None, None, None, None, None, None, 1e-5, 0, None, None) == dlf.DLF_ERR_INVALID_ARG


def test_zero_sized_calls_are_noops():
    d = dlf.conv_desc(0, 8, 8, 16, 16, dtype="bf16")
    dlf.dlf_conv_fused(d, None, None, None, None, None, stream=0)
    g = dlf.gemm_desc(0, 16, 32)
    dlf.dlf_gemm_fused(g, None, None, None, None, None, None, stream=0)
    dlf.dlf_gemm_plain(dlf.gemm_desc(16, 0, 32), None, None, 1.0, None, stream=0)
    dlf.dlf_act_apply(0, "bf16", "relu", None, None, stream=0)
    dlf.dlf_quant_apply(0, None, 1.0, None, stream=0)
    # output smaller than one kernel tap without padding: ho = 0
    dlf.dlf_conv_fused(dlf.conv_desc(1, 2, 2, 8, 8, kh=3, kw=3, pad=0), None, None, None, None, None, stream=0)


def _status(fn, *args):
    return fn(*args)


@fake_pointers
def test_conv_validation_statuses():
    lib = dlf.raw()
    A, B, Y = 0x100000, 0x200000, 0x300000      # fake, aligned, disjoint
    d = dlf.conv_desc(1, 8, 8, 16, 16, dtype="bf16")
    assert lib.dlf_conv_fused(None, A, B, None, None, Y, 0) == dlf.DLF_ERR_INVALID_ARG
    # c_in % 8 != 0 is gathered value by value; an image row of 2^30 values or more is not
    bad = dlf.conv_desc(1, 1, 1 << 27, 12, 16, kh=1, kw=1, pad=0, dtype="bf16")
    assert lib.dlf_conv_fused(ctypes.byref(bad), A, B, None, None, Y, 0) == dlf.DLF_ERR_UNSUPPORTED
    fp8 = dlf.conv_desc(1, 8, 8, 16, 16, dtype="fp8")
    assert lib.dlf_conv_fused(ctypes.byref(fp8), A, B, None, None, Y, 0) == dlf.DLF_ERR_UNSUPPORTED
    neg = dlf.conv_desc(-1, 8, 8, 16, 16)
    assert lib.dlf_conv_fused(ctypes.byref(neg), A, B, None, None, Y, 0) == dlf.DLF_ERR_INVALID_ARG
    zs = dlf.conv_desc(1, 8, 8, 16, 16, stride=0)
    assert lib.dlf_conv_fused(ctypes.byref(zs), A, B, None, None, Y, 0) == dlf.DLF_ERR_INVALID_ARG
    wrong_act = dlf.conv_desc(1, 8, 8, 16, 16, act=7)
    assert lib.dlf_conv_fused(ctypes.byref(wrong_act), A, B, None, None, Y, 0) == dlf.DLF_ERR_INVALID_ARG
    assert lib.dlf_conv_fused(ctypes.byref(d), None, B, None, None, Y, 0) == dlf.DLF_ERR_INVALID_ARG
    assert lib.dlf_conv_fused(ctypes.byref(d), A + 2, B, None, None, Y, 0) == dlf.DLF_ERR_INVALID_ARG
    assert lib.dlf_conv_fused(ctypes.byref(d), A, B, None, None, A + 64, 0) == dlf.DLF_ERR_ALIAS   # y inside x
    assert lib.dlf_conv_fused(ctypes.byref(d), A, B, Y + 16, None, Y, 0) == dlf.DLF_ERR_ALIAS     # bias inside y
    assert lib.dlf_conv_fused(ctypes.byref(d), A, B, None, Y, Y, 0) == dlf.DLF_ERR_ALIAS         # residual == y
    assert "overlaps" in dlf.dlf_last_error()
    relu_plain = dlf.conv_desc(1, 8, 8, 16, 16, act="relu")
    assert lib.dlf_conv_plain(ctypes.byref(relu_plain), A, B, None, Y, 0) == dlf.DLF_ERR_INVALID_ARG


@fake_pointers
def test_gemm_validation_statuses():
    lib = dlf.raw()
    A, B, C = 0x100000, 0x200000, 0x300000
    def g(**kw):
        base = dict(m=64, n=64, k=64, in_dtype="bf16", out_dtype="bf16", act="gelu_tanh", out_inv_scale=1.0)
        base.update(kw)
        return ctypes.byref(dlf.gemm_desc(**base))
    assert lib.dlf_gemm_fused(g(k=60), A, B, None, None, None, C, 0) == dlf.DLF_ERR_UNSUPPORTED      # k % 8
    assert lib.dlf_gemm_fused(g(in_dtype="fp8", out_dtype="fp8", k=72), A, B, None, None, None, C, 0) == \
        dlf.DLF_ERR_UNSUPPORTED                                                                     # k % 16
    assert lib.dlf_gemm_fused(g(in_dtype="fp8", out_dtype="fp8", act="relu"), A, B, None, None, 0x400000, C, 0) == \
        dlf.DLF_ERR_UNSUPPORTED                                                                     # fp8 + residual
    assert lib.dlf_gemm_fused(g(in_dtype="fp8", out_dtype="fp8", act="relu", out_inv_scale=0.0), A, B, None, None,
                              None, C, 0) == dlf.DLF_ERR_INVALID_ARG
    assert lib.dlf_gemm_fused(g(in_dtype="f32", out_dtype="f32"), A, B, None, None, None, C, 0) == \
        dlf.DLF_ERR_UNSUPPORTED
    assert lib.dlf_gemm_fused(g(), A, B, None, None, None, A, 0) == dlf.DLF_ERR_ALIAS
    assert lib.dlf_gemm_fused(g(), A, B, C + 16, None, None, C, 0) == dlf.DLF_ERR_ALIAS
    assert lib.dlf_gemm_fused(g(), A, B, None, 0x400008, None, C, 0) == dlf.DLF_ERR_INVALID_ARG     # misaligned
    assert lib.dlf_gemm_plain(g(), A, B, ctypes.c_float(1.0), C, 0) == dlf.DLF_ERR_INVALID_ARG       # act != none
    assert lib.dlf_gemm_plain(g(in_dtype="fp8", out_dtype="fp8", act="none"), A, B, ctypes.c_float(1.0), C, 0) == \
        dlf.DLF_ERR_UNSUPPORTED


@fake_pointers
def test_gemm_split_validation_statuses():
    """dlf_gemm_fused_split refuses, before any launch, what it cannot store exactly."""
    lib = dlf.raw()
    A, B = 0x100000, 0x200000
    def g(**kw):
        base = dict(m=64, n=96, k=64, in_dtype="bf16", out_dtype="bf16", act="none", out_inv_scale=1.0)
        base.update(kw)
        return ctypes.byref(dlf.gemm_desc(**base))
    def outs(*ptrs):
        return (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
    Q, K, V = 0x300000, 0x400000, 0x500000
    call = lib.dlf_gemm_fused_split
    assert call(g(), A, B, None, None, 0, outs(Q), 0) == dlf.DLF_ERR_INVALID_ARG          # parts < 1
    assert call(g(), A, B, None, None, 3, None, 0) == dlf.DLF_ERR_INVALID_ARG             # outs NULL
    assert call(g(), A, B, None, None, 3, outs(Q, None, V), 0) == dlf.DLF_ERR_INVALID_ARG  # a NULL part
    assert call(g(), A, B, None, None, 3, outs(Q, K + 8, V), 0) == dlf.DLF_ERR_INVALID_ARG  # misaligned part
    assert call(g(n=100), A, B, None, None, 3, outs(Q, K, V), 0) == dlf.DLF_ERR_INVALID_ARG  # n % parts
    assert call(g(n=5 * 16), A, B, None, None, 5, outs(Q, K, V, Q, K), 0) == dlf.DLF_ERR_UNSUPPORTED  # > 4
    assert call(g(n=3 * 12), A, B, None, None, 3, outs(Q, K, V), 0) == dlf.DLF_ERR_UNSUPPORTED  # 24 B rows
    assert call(g(in_dtype="fp8", out_dtype="fp8", n=3 * 8), A, B, None, None, 3, outs(Q, K, V), 0) == \
        dlf.DLF_ERR_UNSUPPORTED                                                               # 8 B fp8 rows
    assert call(g(), A, B, None, None, 3, outs(Q, Q + 16, V), 0) == dlf.DLF_ERR_ALIAS      # parts overlap
    assert call(g(), A, B, None, None, 3, outs(Q, K, A), 0) == dlf.DLF_ERR_ALIAS           # part over A
    assert call(g(m=0), A, B, None, None, 3, outs(Q, K, V), 0) == dlf.DLF_OK              # empty: no launch


@fake_pointers
def test_gemm_gated_validation_statuses():
    lib = dlf.raw()
    A, B, C = 0x100000, 0x200000, 0x300000
    def g(**kw):
        base = dict(m=64, n=96, k=64, in_dtype="bf16", out_dtype="bf16", act="none", out_inv_scale=1.0)
        base.update(kw)
        return ctypes.byref(dlf.gemm_desc(**base))
    call = lib.dlf_gemm_fused_gated
    assert call(None, A, B, None, None, 0, C, 0) == dlf.DLF_ERR_INVALID_ARG                  # no descriptor
    assert call(g(), A, B, None, None, 7, C, 0) == dlf.DLF_ERR_INVALID_ARG                   # unknown gate
    assert call(g(act="relu"), A, B, None, None, 0, C, 0) == dlf.DLF_ERR_INVALID_ARG         # act != NONE
    assert call(g(n=95), A, B, None, None, 0, C, 0) == dlf.DLF_ERR_INVALID_ARG               # odd n
    assert call(g(in_dtype="fp8", out_dtype="fp8", k=64), A, B, None, None, 0, C, 0) == dlf.DLF_ERR_UNSUPPORTED
    assert call(g(k=60), A, B, None, None, 0, C, 0) == dlf.DLF_ERR_UNSUPPORTED               # k % 8
    assert call(g(), A, B, None, None, 0, A, 0) == dlf.DLF_ERR_ALIAS
    assert call(g(), A, B, None, 0x400008, 0, C, 0) == dlf.DLF_ERR_INVALID_ARG               # misaligned
    assert call(g(m=0), A, B, None, None, 2, C, 0) == dlf.DLF_OK


@fake_pointers
def test_eltwise_validation_statuses():
    lib = dlf.raw()
    A, B, C = 0x100000, 0x200000, 0x300000
    assert lib.dlf_bn_apply(4, 8, dlf.DLF_BF16, A, B, B, B, B, ctypes.c_double(-1.0), C, 0) == dlf.DLF_ERR_INVALID_ARG
    assert lib.dlf_bn_apply(4, 8, dlf.DLF_FP8_E4M3, A, B, B, B, B, ctypes.c_double(1e-5), C, 0) == \
        dlf.DLF_ERR_UNSUPPORTED
    assert lib.dlf_bn_apply(4, 8, dlf.DLF_BF16, A, None, B, B, B, ctypes.c_double(1e-5), C, 0) == \
        dlf.DLF_ERR_INVALID_ARG
    assert lib.dlf_bn_apply(64, 8, dlf.DLF_BF16, A, B, B, B, B, ctypes.c_double(1e-5), A + 16, 0) == dlf.DLF_ERR_ALIAS
    assert lib.dlf_scale_shift_apply(4, 8, dlf.DLF_BF16, A, None, None, C, 0) == dlf.DLF_ERR_INVALID_ARG
    assert lib.dlf_add(64, dlf.DLF_F32, A, B, A + 16, 0) == dlf.DLF_ERR_ALIAS
    assert lib.dlf_act_apply(64, dlf.DLF_F32, 9, A, C, 0) == dlf.DLF_ERR_INVALID_ARG
    assert lib.dlf_act_apply(64, dlf.DLF_F32, 1, A, A + 16, 0) == dlf.DLF_ERR_ALIAS
    assert lib.dlf_quant_apply(64, A, ctypes.c_float(float("nan")), C, 0) == dlf.DLF_ERR_INVALID_ARG
    assert lib.dlf_quant_apply(64, A, ctypes.c_float(-1.0), C, 0) == dlf.DLF_ERR_INVALID_ARG
    assert lib.dlf_quant_apply(64, A, ctypes.c_float(1.0), A + 32, 0) == dlf.DLF_ERR_ALIAS
    assert lib.dlf_quant_apply(64, A + 4, ctypes.c_float(1.0), C, 0) == dlf.DLF_ERR_INVALID_ARG


def test_ffn_pack_layout_and_checks():
    """dlf_ffn_pack writes W[32 rb + l % 32][16 s + 8 (l / 32) + e] at
    ((rb * k/16 + s) * 64 + l) * 8 + e: checked element by element on a random matrix."""
    rng = np.random.default_rng(8)
    rows, k = 64, 48
    w = rng.integers(0, 1 << 16, (rows, k), dtype=np.uint16)
    p = dlf.dlf_ffn_pack(w).reshape(-1)
    ks = k // 16
    for rb in range(rows // 32):
        for s in range(ks):
            for lane in range(64):
                for e in range(8):
                    assert p[((rb * ks + s) * 64 + lane) * 8 + e] == w[32 * rb + lane % 32, 16 * s + 8 * (lane // 32) + e]
    lib = dlf.raw()
    buf = np.zeros(64 * 48, np.uint16)
    assert lib.dlf_ffn_pack(48, 48, buf.ctypes.data, buf.ctypes.data) == dlf.DLF_ERR_INVALID_ARG   # rows % 32
    assert lib.dlf_ffn_pack(64, 40, buf.ctypes.data, buf.ctypes.data) == dlf.DLF_ERR_INVALID_ARG   # k % 16
    assert lib.dlf_ffn_pack(64, 48, buf.ctypes.data, buf.ctypes.data) == dlf.DLF_ERR_ALIAS
    assert lib.dlf_ffn_pack(64, 48, None, buf.ctypes.data) == dlf.DLF_ERR_INVALID_ARG
    assert lib.dlf_ffn_pack(0, 48, None, None) == dlf.DLF_OK


@fake_pointers
def test_ffn_validation_statuses():
    lib = dlf.raw()
    X, W1, W2, Y = 0x100000, 0x200000, 0x400000, 0x600000
    fused = lambda d, **kw: lib.dlf_ffn_fused(ctypes.byref(d), kw.get("x", X), W1, None, W2, None,
                                              kw.get("r", None), kw.get("y", Y), 0)
    assert fused(dlf.ffn_desc(64, 640, 3072)) == dlf.DLF_ERR_UNSUPPORTED          # d_model
    assert fused(dlf.ffn_desc(64, 768, 3000)) == dlf.DLF_ERR_UNSUPPORTED          # d_ff % 256
    assert fused(dlf.ffn_desc(64, 768, 3072, dtype="f32")) == dlf.DLF_ERR_UNSUPPORTED
    assert fused(dlf.ffn_desc(64, 768, 3072, act=9)) == dlf.DLF_ERR_INVALID_ARG
    assert fused(dlf.ffn_desc(-1, 768, 3072)) == dlf.DLF_ERR_INVALID_ARG
    assert fused(dlf.ffn_desc(64, 768, 3072), x=X + 8) == dlf.DLF_ERR_INVALID_ARG  # misaligned
    assert fused(dlf.ffn_desc(64, 768, 3072), y=X + 64) == dlf.DLF_ERR_ALIAS       # y inside x
    assert fused(dlf.ffn_desc(64, 768, 3072), r=Y) == dlf.DLF_ERR_ALIAS            # residual == y
    assert fused(dlf.ffn_desc(0, 768, 3072)) == dlf.DLF_OK                         # empty: no launch
    assert lib.dlf_ffn_fused(None, X, W1, None, W2, None, None, Y, 0) == dlf.DLF_ERR_INVALID_ARG


@fake_pointers
def test_ffn_workspace_size_and_checks():
    """The d_ff split's workspace: S m d_model fp32 where the block splits into S parts (below
    16384 tokens, d_model <= 768, fewer than 160 token blocks of 64 from 4096 tokens, else of
    32: as many parts as fit 256 workgroups, at most one a chunk of 256 features), else 0; too
    small, misaligned or overlapping workspaces are refused before any launch."""
    lib = dlf.raw()
    ws = dlf.dlf_ffn_workspace_bytes
    assert ws(dlf.ffn_desc(8192, 768, 3072)) == 2 * 8192 * 768 * 4        # 128 blocks of 64
    assert ws(dlf.ffn_desc(8191, 768, 3072)) == 2 * 8191 * 768 * 4        # 128 blocks of 64
    assert ws(dlf.ffn_desc(4096, 768, 3072)) == 4 * 4096 * 768 * 4        # 64 blocks of 64
    assert ws(dlf.ffn_desc(6000, 768, 3072)) == 2 * 6000 * 768 * 4        # 94 blocks of 64
    assert ws(dlf.ffn_desc(4095, 768, 3072)) == 2 * 4095 * 768 * 4        # 128 blocks of 32
    assert ws(dlf.ffn_desc(1000, 512, 2048)) == 8 * 1000 * 512 * 4        # 32 blocks: 8 parts
    assert ws(dlf.ffn_desc(128, 768, 3072)) == 12 * 128 * 768 * 4         # 4 blocks: 64, at most 12
    assert ws(dlf.ffn_desc(1, 256, 512)) == 2 * 1 * 256 * 4
    for m, dm, dff in ((10240, 768, 3072), (16383, 256, 512), (16384, 768, 3072), (8192, 1024, 4096),
                       (100, 1024, 4096), (8192, 768, 256), (0, 768, 3072)):
        assert ws(dlf.ffn_desc(m, dm, dff)) == 0, (m, dm, dff)
    n = ctypes.c_size_t(7)
    assert lib.dlf_ffn_workspace_bytes(ctypes.byref(dlf.ffn_desc(64, 640, 3072)), ctypes.byref(n)) \
        == dlf.DLF_ERR_UNSUPPORTED and n.value == 0
    assert lib.dlf_ffn_workspace_bytes(ctypes.byref(dlf.ffn_desc(64, 768, 3072)), None) == dlf.DLF_ERR_INVALID_ARG
    X, W1, W2, Y, R, WS = 0x1000000, 0x2000000, 0x4000000, 0x6000000, 0x8000000, 0xA000000
    d = dlf.ffn_desc(8192, 768, 3072)
    need = ws(d)
    run = lambda w, nbytes, d=d: lib.dlf_ffn_fused_ws(ctypes.byref(d), X, W1, None, W2, None, R, Y, w, nbytes, 0)
    assert run(None, 0) == dlf.DLF_ERR_INVALID_ARG               # the split needs its workspace
    assert run(WS, need - 16) == dlf.DLF_ERR_INVALID_ARG         # too small
    assert run(WS + 8, need) == dlf.DLF_ERR_INVALID_ARG          # misaligned
    assert run(Y - 64, need) == dlf.DLF_ERR_ALIAS                # overlaps y
    assert run(R + 4096, need) == dlf.DLF_ERR_ALIAS              # overlaps the residual
    small = dlf.ffn_desc(0, 768, 3072)
    assert run(None, 0, d=small) == dlf.DLF_OK                   # empty: no launch


@fake_pointers
def test_clock_probe_validation_statuses():
    raw = dlf.raw()
    fake = ctypes.c_void_p(0x100000)
    assert raw.dlf_clock_probe(0, 10, fake, None) == dlf.DLF_ERR_INVALID_ARG
    assert raw.dlf_clock_probe(65537, 10, fake, None) == dlf.DLF_ERR_INVALID_ARG
    assert raw.dlf_clock_probe(8, 0, fake, None) == dlf.DLF_ERR_INVALID_ARG
    assert raw.dlf_clock_probe(8, 10, None, None) == dlf.DLF_ERR_INVALID_ARG
    assert raw.dlf_clock_probe(8, 10, ctypes.c_void_p(0x100008), None) == dlf.DLF_ERR_INVALID_ARG


def test_tuning_reload_reads_the_environment():
    # a reload with and without a switch set is harmless on the host (no launch happens)
    os.environ["DLF_TILE"] = "2"
    try:
        dlf.dlf_tuning_reload()
    finally:
        os.environ.pop("DLF_TILE", None)
        dlf.dlf_tuning_reload()
