"""Oracle of a bf16 Conv -> BN -> activation network run under a fusion plan.

TEST INFRASTRUCTURE: only the tests may import it; it shares no code with the library.

The network is evaluated in binary64 from the fp32 masters, with the storage roundings the
method itself defines and nothing else:
  - a chain the plan fuses computes act(conv(x, W') + b' [+ residual]) with the BN folded
    into W' and b' in binary64 and W' rounded once to bf16 ([OPPL] §3.1 and §6.2: fold in
    high precision, then one cast), and only its result is stored (rounded to bf16) -
    the chain's inner tensors never exist ([OPPL] §2.1, [CANN] "three round trips to one");
  - every op outside a chain stores its own result rounded to bf16; an unfused conv uses
    the master weights rounded to bf16.
bf16 rounding is round_bf16 (nearest, ties to even, from binary64 in one step).  The plan is
the oracle's own (oracle.fusion.plan) or an empty one for the unfused network.
"""
from __future__ import annotations

import numpy as np

from . import activation, add, batchnorm, conv2d, fold_bn, round_bf16, widen

_ACTS = {"relu": "relu", "gelu": "gelu_tanh", "gelu_erf": "gelu_erf"}


def forward(graph, params, inputs, plan):
    """graph: node dicts (op, inputs, shape, attrs ...); params: fp32 masters by node index;
    inputs: {input node: bf16 bit patterns (uint16)}; plan: groups with "nodes".
    Returns {node: binary64 array} for every tensor the plan keeps in memory."""
    group_of = {i: g for g in plan for i in g["nodes"]}
    vals = {}
    for i, nd in enumerate(graph):
        op = nd["op"]
        g = group_of.get(i)
        if op == "input":
            vals[i] = widen(inputs[i], "bf16")
            continue
        if g is not None:
            if g["nodes"][-1] != i:
                continue                                   # inside a fused chain
            vals[i] = _fused(graph, params, vals, g["nodes"])
            continue
        src = [vals[j] for j in nd["inputs"]]
        if op == "conv":
            a = nd["attrs"]
            w = round_bf16(params[i]["w"].astype(np.float64))
            y = conv2d(src[0], w, None, a["stride"], a["pad"])
        elif op == "batchnorm":
            p = params[i]
            y = batchnorm(src[0], p["gamma"], p["beta"], p["mean"], p["var"], nd["attrs"]["eps"])
        elif op == "add":
            y = add(src[0], src[1])
        elif op in _ACTS:
            y = activation(src[0], _ACTS[op])
        else:
            raise NotImplementedError(op)
        vals[i] = round_bf16(y)
    return vals


def _fused(graph, params, vals, nodes):
    c = nodes[0]
    a = graph[c]["attrs"]
    w = params[c]["w"]
    rest = nodes[1:]
    b = None
    if rest and graph[rest[0]]["op"] == "batchnorm":
        p = params[rest[0]]
        w, b = fold_bn(w, None, p["gamma"], p["beta"], p["mean"], p["var"], graph[rest[0]]["attrs"]["eps"])
        rest = rest[1:]
    w = round_bf16(np.asarray(w, dtype=np.float64))
    y = conv2d(vals[graph[c]["inputs"][0]], w, b, a["stride"], a["pad"])
    prev = nodes[nodes.index(rest[0]) - 1] if rest else c
    for i in rest:
        op = graph[i]["op"]
        if op == "add":
            other = [j for j in graph[i]["inputs"] if j != prev][0]
            y = add(y, vals[other])
        elif op in _ACTS:
            y = activation(y, _ACTS[op])
        else:
            raise NotImplementedError(op)
        prev = i
    return round_bf16(y)
