"""Seeded synthetic workloads for the fused Conv/MatMul -> BatchNorm -> activation operator.

This module is shared by the HIP path's callers (tests, bench, smoke) and by the
CPU oracle's callers.  It only *draws* inputs: it holds none of the operator's
arithmetic (no convolution, no normalisation, no folding, no activation and no
fp8 codec of its own).  Storage-format casts of the drawn values use PyTorch's
CPU casts (float32 -> bfloat16 and float32 -> float8_e4m3fn, both round to
nearest even), exactly as a model loader would store them.

The five named workloads follow the configurations the fused operator is
measured on: a small fp32 conv, two bf16 ResNet-stage 3x3 convs, the LLaMA-7B
FFN up-projection shape with bias + GELU(tanh), and an fp8 e4m3 GEMM with a
static-scale epilogue.  Every random draw comes from numpy's PCG64 generator
seeded with the workload's index, in a fixed order:
x, W, conv bias, gamma, beta, mean, var, stressed-channel choice, residual,
GEMM bias.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = [
    "ConvWorkload", "GemmWorkload", "Fp8GemmWorkload", "FfnWorkload", "FFN_BERT_BASE", "WORKLOADS",
    "generate", "bf16_bits", "e4m3_codes", "workload",
]


@dataclass(frozen=True)
class ConvWorkload:
    """Conv2d (NHWC activations, OHWI weights) + BatchNorm + [residual] + activation."""
    name: str
    dtype: str                 # "f32" or "bf16": storage type of x, residual and y
    n: int
    h: int
    w: int
    cin: int
    cout: int
    kh: int = 3
    kw: int = 3
    stride: int = 1
    pad: int = 1
    conv_bias: bool = False
    eps: float = 1e-5
    act: str = "relu"          # "none" | "relu" | "gelu_tanh"
    residual: bool = False
    stress_frac: float = 0.0   # fraction of channels whose running var ~ U(1e-6, 1e-3)
    seed: int = 0

    @property
    def ho(self) -> int:
        return (self.h + 2 * self.pad - self.kh) // self.stride + 1

    @property
    def wo(self) -> int:
        return (self.w + 2 * self.pad - self.kw) // self.stride + 1

    @property
    def gemm_mnk(self):
        return self.n * self.ho * self.wo, self.cout, self.kh * self.kw * self.cin

    @property
    def kind(self) -> str:
        return "conv"


@dataclass(frozen=True)
class GemmWorkload:
    """MatMul (a 1x1 conv over tokens): y = x W^T + bias, then activation; bf16 in/out."""
    name: str
    m: int
    n: int
    k: int
    act: str = "gelu_tanh"
    bias: bool = True
    dtype: str = "bf16"
    seed: int = 3

    @property
    def gemm_mnk(self):
        return self.m, self.n, self.k

    @property
    def kind(self) -> str:
        return "gemm"


@dataclass(frozen=True)
class Fp8GemmWorkload:
    """fp8 e4m3 MatMul with static per-tensor scales, per-channel norm scale/shift,
    ReLU and static per-tensor e4m3 output quantisation."""
    name: str
    m: int
    n: int
    k: int
    eps: float = 1e-5
    out_scale: float = 8.0     # static output scale s_y, fixed ahead of time (a power of two)
    seed: int = 4

    @property
    def gemm_mnk(self):
        return self.m, self.n, self.k

    @property
    def kind(self) -> str:
        return "fp8gemm"

    @property
    def dtype(self) -> str:
        return "fp8"


@dataclass(frozen=True)
class FfnWorkload:
    """Transformer feed-forward block: y = act(x W1^T + b1) W2^T + b2 [+ residual]; bf16
    tensors, fp32 biases.  W1 is [d_ff][d_model], W2 is [d_model][d_ff] (the [out][in] layout
    of a linear layer)."""
    name: str
    m: int
    d_model: int
    d_ff: int
    act: str = "gelu_tanh"
    residual: bool = True
    seed: int = 5

    @property
    def kind(self) -> str:
        return "ffn"

    @property
    def dtype(self) -> str:
        return "bf16"


# BERT-base's feed-forward block (d_model 768, d_ff 3072) over 64 sequences of 128 tokens
FFN_BERT_BASE = FfnWorkload("ffn_bf16_8192x768x3072_bias_gelu_tanh_residual", 8192, 768, 3072)


WORKLOADS = {
    0: ConvWorkload("conv3x3_f32_n1_32x32_16to32_bias_bn_relu", "f32", 1, 32, 32, 16, 32,
                    conv_bias=True, eps=1e-5, act="relu", seed=0),
    1: ConvWorkload("conv3x3_bf16_n32_56x56_64to64_bn_relu", "bf16", 32, 56, 56, 64, 64,
                    conv_bias=False, eps=1e-5, act="relu", seed=1),
    2: ConvWorkload("conv3x3_bf16_n32_14x14_256to256_bn_residual_relu", "bf16", 32, 14, 14, 256, 256,
                    conv_bias=False, eps=1e-2, act="relu", residual=True, stress_frac=0.1, seed=2),
    3: GemmWorkload("matmul_bf16_4096x11008x4096_bias_gelu_tanh", 4096, 11008, 4096, seed=3),
    4: Fp8GemmWorkload("matmul_fp8e4m3_8192x4096x4096_scale_shift_relu_quant", 8192, 4096, 4096, seed=4),
}


def workload(index: int, **overrides):
    """The named workload `index`, optionally with fields replaced (e.g. smaller shapes)."""
    base = WORKLOADS[index]
    return dataclasses.replace(base, **overrides) if overrides else base


def bf16_bits(a32: np.ndarray) -> np.ndarray:
    """Store float32 values as bfloat16 (PyTorch's RNE cast); returns the uint16 bit patterns."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def e4m3_codes(a32: np.ndarray) -> np.ndarray:
    """Store float32 values (|v| <= 448) as OCP e4m3fn codes (PyTorch's RNE cast)."""
    import torch
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    if a32.size and float(np.max(np.abs(a32))) >= 464.0:
        raise ValueError("value outside the e4m3 range handed to the storage cast")
    t = torch.from_numpy(a32).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def _store(dtype: str, a32: np.ndarray) -> np.ndarray:
    return a32 if dtype == "f32" else bf16_bits(a32)


def _bn_params(rng, c: int, stress_frac: float):
    gamma = rng.uniform(0.5, 1.5, c).astype(np.float32)
    beta = rng.normal(0.0, 0.1, c).astype(np.float32)
    mean = rng.normal(0.0, 0.1, c).astype(np.float32)
    var = rng.uniform(0.01, 1.0, c)
    stressed = np.zeros(0, dtype=np.int64)
    if stress_frac > 0.0:
        stressed = np.sort(rng.choice(c, int(round(stress_frac * c)), replace=False))
        var[stressed] = rng.uniform(1e-6, 1e-3, stressed.size)
    return gamma, beta, mean, var.astype(np.float32), stressed


def generate(wl) -> dict:
    """Draw every input of workload `wl` (seeded, deterministic).

    Returned arrays are host numpy arrays in their storage format:
    float32 values, bf16 bit patterns (uint16) or e4m3 codes (uint8).
    Model parameters (W, conv bias, gamma, beta, mean, var) are float32 masters.
    """
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    out: dict = {"workload": wl}
    if isinstance(wl, ConvWorkload):
        x = rng.standard_normal((wl.n, wl.h, wl.w, wl.cin)).astype(np.float32)
        fan_in = wl.cin * wl.kh * wl.kw
        w = rng.normal(0.0, np.sqrt(2.0 / fan_in), (wl.cout, wl.kh, wl.kw, wl.cin)).astype(np.float32)
        b = rng.normal(0.0, 0.1, wl.cout).astype(np.float32) if wl.conv_bias else None
        gamma, beta, mean, var, stressed = _bn_params(rng, wl.cout, wl.stress_frac)
        res = None
        if wl.residual:
            res = _store(wl.dtype, rng.standard_normal((wl.n, wl.ho, wl.wo, wl.cout)).astype(np.float32))
        out.update(x=_store(wl.dtype, x), w=w, conv_bias=b, gamma=gamma, beta=beta, mean=mean,
                   var=var, eps=float(wl.eps), residual=res, stressed=stressed)
    elif isinstance(wl, GemmWorkload):
        x = rng.standard_normal((wl.m, wl.k)).astype(np.float32)
        w = rng.normal(0.0, 1.0 / np.sqrt(max(wl.k, 1)), (wl.n, wl.k)).astype(np.float32)
        bias = rng.normal(0.0, 0.02, wl.n).astype(np.float32) if wl.bias else None
        out.update(x=bf16_bits(x), w=bf16_bits(w), bias=bias)
    elif isinstance(wl, Fp8GemmWorkload):
        x = rng.standard_normal((wl.m, wl.k)).astype(np.float32)
        w = rng.standard_normal((wl.n, wl.k)).astype(np.float32)
        gamma, beta, mean, var, _ = _bn_params(rng, wl.n, 0.0)
        s_x = np.float32(float(np.max(np.abs(x))) / 448.0) if x.size else np.float32(1.0)
        s_w = np.float32(float(np.max(np.abs(w))) / 448.0) if w.size else np.float32(1.0)
        xq = e4m3_codes((x.astype(np.float64) / float(s_x)).astype(np.float32))
        wq = e4m3_codes((w.astype(np.float64) / float(s_w)).astype(np.float32))
        out.update(x=xq, w=wq, s_x=float(s_x), s_w=float(s_w), gamma=gamma, beta=beta, mean=mean,
                   var=var, eps=float(wl.eps), conv_bias=None, s_y=float(np.float32(wl.out_scale)))
    elif isinstance(wl, FfnWorkload):
        x = rng.standard_normal((wl.m, wl.d_model)).astype(np.float32)
        w1 = rng.normal(0.0, 1.0 / np.sqrt(max(wl.d_model, 1)), (wl.d_ff, wl.d_model)).astype(np.float32)
        b1 = rng.normal(0.0, 0.02, wl.d_ff).astype(np.float32)
        w2 = rng.normal(0.0, 1.0 / np.sqrt(max(wl.d_ff, 1)), (wl.d_model, wl.d_ff)).astype(np.float32)
        b2 = rng.normal(0.0, 0.02, wl.d_model).astype(np.float32)
        res = bf16_bits(rng.standard_normal((wl.m, wl.d_model)).astype(np.float32)) if wl.residual else None
        out.update(x=bf16_bits(x), w1=bf16_bits(w1), b1=b1, w2=bf16_bits(w2), b2=b2, residual=res)
    else:
        raise TypeError(f"unknown workload type {type(wl)!r}")
    return out
