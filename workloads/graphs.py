"""Seeded synthetic graphs for the host fusion pass and the network runs.

Like the rest of this package it only draws inputs: graph structure, shapes, per-node
operation counts and parameters.  It holds none of the pass's logic and none of the
operator's arithmetic.

A graph is a list of node dicts in topological order (the format the fusion pass takes):
  op, inputs, shape, dtype, flops, output, training
plus, for the nodes a network run executes, "attrs" (conv geometry, BN epsilon).
Shapes are NHWC for convolutions and [rows, features] for MatMuls.
"""
from __future__ import annotations

from typing import List

import numpy as np

__all__ = ["resnet_stage_graph", "stem_graph", "random_graph", "draw_params"]


class _Builder:
    def __init__(self, dtype: str):
        self.nodes: List[dict] = []
        self.dtype = dtype

    def add(self, op, inputs, shape, flops=0, dtype=None, **attrs) -> int:
        self.nodes.append(dict(op=op, inputs=list(inputs), shape=tuple(int(s) for s in shape),
                               dtype=dtype or self.dtype, flops=int(flops), output=False,
                               training=False, attrs=attrs))
        return len(self.nodes) - 1

    def conv(self, x, cout, k, stride, pad):
        n, h, w, cin = self.nodes[x]["shape"]
        ho = (h + 2 * pad - k) // stride + 1
        wo = (w + 2 * pad - k) // stride + 1
        return self.add("conv", [x], (n, ho, wo, cout), 2 * n * ho * wo * cout * k * k * cin,
                        kh=k, kw=k, stride=stride, pad=pad, cin=cin, cout=cout)

    def bn(self, x, eps=1e-5):
        shp = self.nodes[x]["shape"]
        return self.add("batchnorm", [x], shp, 2 * int(np.prod(shp)), eps=eps)

    def ew(self, op, inputs):
        shp = self.nodes[inputs[0]]["shape"]
        return self.add(op, inputs, shp, int(np.prod(shp)))


def stem_graph(n=32, h=224, w=224, dtype="bf16"):
    """ResNet stem: 7x7 stride-2 pad-3 conv over 3 input channels -> BN -> ReLU."""
    b = _Builder(dtype)
    x = b.add("input", [], (n, h, w, 3))
    y = b.ew("relu", [b.bn(b.conv(x, 64, 7, 2, 3))])
    b.nodes[y]["output"] = True
    return b.nodes


def resnet_stage_graph(n=32, h=56, w=56, cin=256, cmid=128, cout=512, stride=2, blocks=2,
                       dtype="bf16"):
    """Bottleneck blocks of a ResNet stage: 1x1 -> BN -> ReLU -> 3x3 (stride on the first
    block) -> BN -> ReLU -> 1x1 -> BN -> Add(shortcut) -> ReLU.  The first block's shortcut is
    a strided 1x1 conv + BN (a downsample branch competing for the Add), the others the
    block input itself."""
    b = _Builder(dtype)
    x = b.add("input", [], (n, h, w, cin))
    for blk in range(blocks):
        s = stride if blk == 0 else 1
        y = b.ew("relu", [b.bn(b.conv(x, cmid, 1, 1, 0))])
        y = b.ew("relu", [b.bn(b.conv(y, cmid, 3, s, 1))])
        y = b.bn(b.conv(y, cout, 1, 1, 0))
        if blk == 0 and (s != 1 or b.nodes[x]["shape"][3] != cout):
            sc = b.bn(b.conv(x, cout, 1, s, 0))
        else:
            sc = x
        x = b.ew("relu", [b.ew("add", [y, sc])])
    b.nodes[x]["output"] = True
    return b.nodes


_OPS = ["conv", "matmul", "matmul_fp8", "bias_add", "batchnorm", "add", "relu", "gelu",
        "gelu_erf", "quant", "reshape"]


def random_graph(seed: int, n_nodes: int = 14) -> List[dict]:
    """A random DAG over the pass's vocabulary, biased towards chains (each node reads the
    previous one with probability 0.8) and towards shapes that agree, so that every legality
    check of the pass meets both outcomes.  Structure only: no attrs."""
    rng = np.random.default_rng(seed)
    shapes = [(4, 8), (4, 16)]
    dtypes = ["bf16", "bf16", "bf16", "f32"]
    nodes = [dict(op="input", inputs=[], shape=shapes[0], dtype="bf16", flops=0, output=False,
                  training=False)]
    later = {"conv": 0, "matmul": 0, "matmul_fp8": 0, "bias_add": 1, "batchnorm": 1, "add": 2,
             "relu": 3, "gelu": 3, "gelu_erf": 3}
    epi = [(0, "bias_add"), (0, "batchnorm"), (1, "add"), (2, "relu"), (2, "gelu"), (2, "gelu_erf"),
           (3, "quant")]
    for i in range(1, n_nodes):
        op = _OPS[int(rng.integers(len(_OPS)))]
        if rng.random() < 0.25:
            op = "input"
        prev = i - 1 if rng.random() < 0.8 else int(rng.integers(i))
        if nodes[prev]["op"] in later and rng.random() < 0.75:
            # continue an epilogue in pattern order
            nxt = [o for st, o in epi if st >= later[nodes[prev]["op"]]]
            op = nxt[int(rng.integers(len(nxt)))]
        inputs = [] if op == "input" else [prev]
        if op == "add":
            same = [j for j in range(i) if nodes[j]["shape"] == nodes[prev]["shape"]
                    and nodes[j]["dtype"] == nodes[prev]["dtype"]]
            other = same[int(rng.integers(len(same)))] if rng.random() < 0.7 else int(rng.integers(i))
            inputs.append(other)
            if rng.random() < 0.5:
                inputs.reverse()
        shape = shapes[int(rng.integers(2))] if op in ("input", "reshape") or rng.random() < 0.15 \
            else nodes[prev]["shape"]
        dtype = dtypes[int(rng.integers(len(dtypes)))] if op == "input" or rng.random() < 0.1 \
            else nodes[prev]["dtype"]
        if op == "quant":
            dtype = "fp8"
        flops = int(rng.integers(0, 1 << 20)) if op in ("conv", "matmul", "matmul_fp8") \
            else int(rng.integers(0, 64))
        nodes.append(dict(op=op, inputs=inputs, shape=shape, dtype=dtype, flops=flops,
                          output=bool(rng.random() < 0.1), training=bool(op == "batchnorm" and rng.random() < 0.2)))
    return nodes


def draw_params(graph: List[dict], seed: int) -> dict:
    """Seeded fp32 parameters for every conv and BN node of a network graph, and the graph's
    inputs: conv weights OHWI ~ N(0, 1/sqrt(fan_in)), no conv bias; BN gamma ~ U(0.5, 1.5),
    beta ~ N(0, 0.1), mean ~ N(0, 0.1), var ~ U(0.5, 1.5); inputs ~ N(0, 1).  Returned as
    fp32 arrays keyed by node index (the storage casts belong to the caller)."""
    rng = np.random.default_rng(seed)
    out = {}
    for i, nd in enumerate(graph):
        if nd["op"] == "input":
            out[i] = {"x": rng.standard_normal(nd["shape"]).astype(np.float32)}
        elif nd["op"] == "conv":
            a = nd["attrs"]
            fan = a["kh"] * a["kw"] * a["cin"]
            w = rng.standard_normal((a["cout"], a["kh"], a["kw"], a["cin"])) / np.sqrt(fan)
            out[i] = {"w": w.astype(np.float32)}
        elif nd["op"] == "batchnorm":
            c = nd["shape"][-1]
            out[i] = {"gamma": rng.uniform(0.5, 1.5, c).astype(np.float32),
                      "beta": (0.1 * rng.standard_normal(c)).astype(np.float32),
                      "mean": (0.1 * rng.standard_normal(c)).astype(np.float32),
                      "var": rng.uniform(0.5, 1.5, c).astype(np.float32)}
    return out
