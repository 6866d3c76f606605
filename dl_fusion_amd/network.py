"""A Conv -> BN -> activation network run through the C ABI under the library's fusion plan.

The host pass (dlf_fusion_plan) chooses which chains become one launch; at load time each
chosen chain's BatchNorm is folded into its conv (dlf_fold_bn, binary64, one rounding to
bf16) and every tensor the plan keeps in memory gets its buffer.  forward() then only
enqueues kernels: one dlf_conv_fused per chosen chain, and the separate conv / BN / Add /
activation kernels for every op outside a chain.  With fuse=False every op runs on its own,
which is the unfused network the fused one is measured against.  A chain the library answers
with DLF_ERR_UNSUPPORTED (it launches nothing then) runs as its separate ops instead, through
buffers of its own for the chain's inner tensors, from that call on ("OpenPPL算子融合深度解析"
§4.2; the MindIE-SD RFC §3.7 falls back to the original graph).

The graph format is the pass's (a list of node dicts in topological order: op, inputs,
shape, dtype, flops, output, training, plus "attrs" with conv geometry and BN epsilon);
parameters are fp32 masters keyed by node index (conv "w" in OHWI; BN gamma, beta, mean,
var).  bf16 networks of conv, batchnorm, add, relu, gelu and gelu_erf nodes are executed.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (DLF_ERR_UNSUPPORTED, DlfError, conv_desc, dlf_act_apply, dlf_add, dlf_bn_apply, dlf_conv_fused,
               dlf_conv_plain, dlf_fold_bn, dlf_fusion_plan)

# MI355X: dense bf16 peak over HBM bandwidth (flops per byte), and the autofusion article's
# fraction of a group's arithmetic charged as the cost of the bigger kernel
RIDGE_BF16 = 2516.6e12 / 8.0e12
OVERHEAD_FRAC = 0.05
_ACTS = {"relu": "relu", "gelu": "gelu_tanh", "gelu_erf": "gelu_erf"}


def _bf16_bits(w: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _dev_bf16(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def _dev_f32(a, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class Network:
    def __init__(self, graph, params, fuse=True, ridge=RIDGE_BF16, overhead_frac=OVERHEAD_FRAC,
                 device="cuda"):
        for i, nd in enumerate(graph):
            if nd["dtype"] != "bf16":
                raise NotImplementedError(f"node {i}: the network runner executes bf16 graphs")
            if nd["op"] not in ("input", "conv", "batchnorm", "add") and nd["op"] not in _ACTS:
                raise NotImplementedError(f"node {i}: op {nd['op']} is not executed here")
            if nd["op"] == "batchnorm" and nd.get("training", False):
                raise NotImplementedError(f"node {i}: a BatchNorm in training mode (batch statistics) is not executed here")
        self.graph = graph
        self.plan = dlf_fusion_plan(graph, ridge, overhead_frac) if fuse else []
        self.saved_bytes = sum(g["saved"] for g in self.plan)
        group_of = {i: g for g in self.plan for i in g["nodes"]}
        self.bufs = {}
        for i, nd in enumerate(graph):
            g = group_of.get(i)
            if nd["op"] == "input" or (g is not None and g["nodes"][-1] != i):
                continue                       # bound at run time, or kept in registers
            self.bufs[i] = torch.empty(nd["shape"], dtype=torch.bfloat16, device=device)
        self.inputs = [i for i, nd in enumerate(graph) if nd["op"] == "input"]
        self.outputs = [i for i, nd in enumerate(graph) if nd.get("output")]
        self.launches = 0
        self._steps = []
        for i, nd in enumerate(graph):
            g = group_of.get(i)
            if g is not None:
                if g["nodes"][-1] == i:
                    self._steps.append(self._fused_step(g, params, device))
                    self.launches += 1
            elif nd["op"] != "input":
                self._steps.append(self._single_step(i, params, device))
                self.launches += 1

    # ---- load time ----------------------------------------------------------------------
    def _conv_geometry(self, c, act):
        nd = self.graph[c]
        a = nd["attrs"]
        n, h, w, cin = self.graph[nd["inputs"][0]]["shape"]
        return conv_desc(n, h, w, cin, a["cout"], a["kh"], a["kw"], a["stride"], a["pad"], "bf16", act)

    def _fused_step(self, g, params, device):
        nodes = g["nodes"]
        c = nodes[0]
        if self.graph[c]["op"] != "conv":
            raise NotImplementedError("fused chains are headed by a conv here")
        bn = next((i for i in nodes if self.graph[i]["op"] == "batchnorm"), None)
        add = next((i for i in nodes if self.graph[i]["op"] == "add"), None)
        act = next((_ACTS[self.graph[i]["op"]] for i in nodes if self.graph[i]["op"] in _ACTS), "none")
        if any(self.graph[i]["op"] == "bias_add" for i in nodes):
            raise NotImplementedError("conv networks carry no BiasAdd")
        w = params[c]["w"]
        if bn is not None:
            p = params[bn]
            w_bits, bias = dlf_fold_bn(w, None, p["gamma"], p["beta"], p["mean"], p["var"],
                                       self.graph[bn]["attrs"]["eps"], "bf16")
            bias_d = _dev_f32(bias, device)
        else:
            w_bits, bias_d = _bf16_bits(w), None
        w_d = _dev_bf16(w_bits, device)
        desc = self._conv_geometry(c, act)
        x_src = self.graph[c]["inputs"][0]
        res_src = None
        if add is not None:
            prev = nodes[nodes.index(add) - 1]
            res_src = [j for j in self.graph[add]["inputs"] if j != prev][0]
        out = nodes[-1]
        fallback = []            # the chain's separate ops and its inner buffers, once needed

        def run(env, stream):
            if not fallback:
                res = env[res_src] if res_src is not None else None
                try:
                    dlf_conv_fused(desc, env[x_src], w_d, bias_d, res, env[out], stream)
                    return
                except DlfError as e:
                    if e.status != DLF_ERR_UNSUPPORTED:
                        raise
                    inner = {i: torch.empty(self.graph[i]["shape"], dtype=torch.bfloat16, device=device)
                             for i in nodes[:-1]}
                    fallback.append(([self._single_step(i, params, device) for i in nodes], inner))
            steps, inner = fallback[0]
            local = dict(env)
            local.update(inner)
            for st in steps:
                st(local, stream)
        return run

    def _single_step(self, i, params, device):
        nd = self.graph[i]
        op = nd["op"]
        src = nd["inputs"]
        if op == "conv":
            desc = self._conv_geometry(i, "none")
            w_d = _dev_bf16(_bf16_bits(params[i]["w"]), device)

            def run(env, stream):
                dlf_conv_plain(desc, env[src[0]], w_d, None, env[i], stream)
        elif op == "batchnorm":
            p = [_dev_f32(params[i][k], device) for k in ("gamma", "beta", "mean", "var")]
            c = nd["shape"][-1]
            rows = int(np.prod(nd["shape"])) // c
            eps = nd["attrs"]["eps"]

            def run(env, stream):
                dlf_bn_apply(rows, c, "bf16", env[src[0]], *p, eps, env[i], stream)
        elif op == "add":
            count = int(np.prod(nd["shape"]))

            def run(env, stream):
                dlf_add(count, "bf16", env[src[0]], env[src[1]], env[i], stream)
        else:
            count = int(np.prod(nd["shape"]))
            act = _ACTS[op]

            def run(env, stream):
                dlf_act_apply(count, "bf16", act, env[src[0]], env[i], stream)
        return run

    # ---- run time -----------------------------------------------------------------------
    def forward(self, inputs, stream=None):
        """inputs: {input node index: bf16 device tensor}.  Enqueues every launch on the
        stream and returns {output node index: bf16 device tensor} (the network's buffers)."""
        env = dict(self.bufs)
        for i in self.inputs:
            t = inputs[i]
            if tuple(t.shape) != tuple(self.graph[i]["shape"]) or t.dtype != torch.bfloat16:
                raise ValueError(f"input {i}: expected bf16 {self.graph[i]['shape']}")
            env[i] = t
        for step in self._steps:
            step(env, stream)
        return {i: env[i] for i in self.outputs}
