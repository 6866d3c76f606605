"""Oracle of a bf16 Conv -> BN -> activation network run under a fusion plan.

TEST INFRASTRUCTURE: only the tests may import it; it shares no code with the library.

Every step is the plain definition in binary64, from the fp32 masters, with no folding:
  - a chain the plan fuses is conv (master weights) -> BN -> [+ residual] -> activation, and
    only its result is a stored tensor - the chain's inner tensors never exist ([OPPL] §2.1,
    [CANN] "three round trips to one"); folding is an identity of this composition ([OPPL]
    §3.1), so it does not appear here;
  - every op outside a chain is its own step and stores its own result.
A network keeps its stored tensors in bf16, so forward() rounds each stored result once to
bf16 (round_bf16: nearest, ties to even, from binary64 in one step) before later steps read
it.  step() evaluates one step on given stored inputs without that rounding: the per-layer
parity check feeds it the GPU's own stored tensors.
"""
from __future__ import annotations

import numpy as np

from . import activation, add, batchnorm, conv2d, round_bf16, widen

_ACTS = {"relu": "relu", "gelu": "gelu_tanh", "gelu_erf": "gelu_erf"}


def step(graph, params, vals, nodes, with_pre=False):
    """The stored tensor that the step `nodes` (a fused chain in chain order, or [i] for an op
    on its own) produces, in binary64 and unrounded, from the stored tensors in `vals`
    ({node: binary64 array}).  with_pre: returns (pre, out), pre being the value the step's
    activation is applied to (out itself for a step that ends in no activation)."""
    head = nodes[0]
    nd = graph[head]
    op = nd["op"]
    src = [vals[j] for j in nd["inputs"]]
    if op == "conv":
        a = nd["attrs"]
        y = conv2d(src[0], np.asarray(params[head]["w"], dtype=np.float64), None, a["stride"], a["pad"])
    elif op == "batchnorm":
        p = params[head]
        y = batchnorm(src[0], p["gamma"], p["beta"], p["mean"], p["var"], nd["attrs"]["eps"])
    elif op == "add":
        y = add(src[0], src[1])
    elif op in _ACTS:
        pre = src[0]
        y = activation(src[0], _ACTS[op])
    else:
        raise NotImplementedError(op)
    if op not in _ACTS:
        pre = y
    prev = head
    for i in nodes[1:]:
        op = graph[i]["op"]
        if op == "batchnorm":
            p = params[i]
            y = batchnorm(y, p["gamma"], p["beta"], p["mean"], p["var"], graph[i]["attrs"]["eps"])
        elif op == "add":
            other = [j for j in graph[i]["inputs"] if j != prev][0]
            y = add(y, vals[other])
        elif op in _ACTS:
            pre = y
            y = activation(y, _ACTS[op])
        else:
            raise NotImplementedError(op)
        if op not in _ACTS:
            pre = y
        prev = i
    return (pre, y) if with_pre else y


def steps(graph, plan):
    """The steps of the network under `plan`, in execution order: {stored node: nodes}."""
    group_of = {i: g for g in plan for i in g["nodes"]}
    out = {}
    for i, nd in enumerate(graph):
        if nd["op"] == "input":
            continue
        g = group_of.get(i)
        if g is None:
            out[i] = [i]
        elif g["nodes"][-1] == i:
            out[i] = list(g["nodes"])
    return out


def forward(graph, params, inputs, plan):
    """graph: node dicts (op, inputs, shape, attrs ...); params: fp32 masters by node index;
    inputs: {input node: bf16 bit patterns (uint16)}; plan: groups with "nodes".
    Returns {node: binary64 array} for every tensor the plan keeps in memory, each rounded to
    bf16 as it is stored."""
    vals = {i: widen(inputs[i], "bf16") for i, nd in enumerate(graph) if nd["op"] == "input"}
    for j, nodes in steps(graph, plan).items():
        vals[j] = round_bf16(step(graph, params, vals, nodes))
    return vals
