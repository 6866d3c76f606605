"""Oracle of the host fusion pass: which Conv/MatMul -> BN -> activation chains of a graph
become one fused launch.

TEST INFRASTRUCTURE, like the rest of this package: only the tests may import it.  It shares
no code with the library's pass (``fusion_pass.cpp``) and never calls it.

The pass follows the three stages of the CANN graph-autofusion article ([CANN], the
aitangshan.cn page: pattern matching, benefit estimation, conflict resolution), with the
legality checks of [OPPL] §4.1-§4.2 (a fused intermediate has exactly one consumer, the BN
is in inference mode, the residual of an epilogue Add is a tensor of the same shape, no
broadcast).  Pure Python over small graphs, written for reading, not speed.

Graph: a list of nodes in topological order; each node is a dict
  op        "input" | "conv" | "matmul" | "matmul_fp8" | "bias_add" | "batchnorm" | "add"
            | "relu" | "gelu" | "gelu_erf" | "quant" | anything else (never fused)
  inputs    list of producer indices (each smaller than the node's own index)
  shape     output shape (tuple of ints)
  dtype     output storage type: "f32" | "bf16" | "fp8"
  flops     arithmetic of the node as the caller counts it (int)
  output    True when the tensor is a graph output (it must reach memory)
  training  True for a BatchNorm in training mode (never folded)
"""
from __future__ import annotations

from typing import Dict, List, Sequence

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
CONTRACTIONS = ("conv", "matmul", "matmul_fp8")
ACTIVATIONS = ("relu", "gelu", "gelu_erf")

# MI355X dense bf16 peak over HBM bandwidth: the flops the chip does in the time it moves a
# byte (2516.6 TFLOP/s / 8 TB/s)
DEFAULT_RIDGE = 2516.6e12 / 8.0e12
DEFAULT_OVERHEAD_FRAC = 0.05


def tensor_bytes(node: dict) -> int:
    n = 1
    for d in node["shape"]:
        n *= int(d)
    return n * ELEM_BYTES[node["dtype"]]


def consumers(graph: Sequence[dict]) -> List[List[int]]:
    """For every node, the nodes that read its output (one entry per input slot)."""
    out: List[List[int]] = [[] for _ in graph]
    for i, nd in enumerate(graph):
        for j in nd["inputs"]:
            out[j].append(i)
    return out


# ---- stage 1: pattern matching ----------------------------------------------------------
#
# The pattern library is the epilogue the fused kernels carry, in its fixed order
# (bias/BN -> residual -> activation -> quantisation, [OPPL] §4.3, [RFC] §3.4):
#
#   contraction  [bias_add | batchnorm]  [add]  [activation]  [quant]
#
# with at least one op after the contraction.  Quantisation closes only chains headed by
# the fp8 MatMul, and that chain takes no residual.  Every match, the short ones included,
# is a candidate: a chain cut short by a conflict at stage 3 is then still on the list.

_STAGE = {"bias_add": 0, "batchnorm": 0, "add": 1, "quant": 3}
for _a in ACTIVATIONS:
    _STAGE[_a] = 2


def _step_ok(graph, chain: List[int], nxt: int) -> bool:
    """May node nxt extend the chain (whose last node produces its input)?"""
    head = graph[chain[0]]
    last = graph[chain[-1]]
    nd = graph[nxt]
    op = nd["op"]
    if op not in _STAGE:
        return False
    prev_stage = -1 if len(chain) == 1 else _STAGE[last["op"]]
    if _STAGE[op] <= prev_stage:
        return False
    if tuple(nd["shape"]) != tuple(head["shape"]):
        return False
    if op == "batchnorm" and nd.get("training", False):
        return False
    if op == "add":
        if head["op"] == "matmul_fp8" or len(nd["inputs"]) != 2 or nd["dtype"] != head["dtype"]:
            return False
        other = [j for j in nd["inputs"] if j != chain[-1]]
        if len(other) != 1:                      # x + x: both slots read the chain value
            return False
        r = graph[other[0]]
        return tuple(r["shape"]) == tuple(nd["shape"]) and r["dtype"] == nd["dtype"]
    if len(nd["inputs"]) != 1:
        return False
    if op == "quant":
        return head["op"] == "matmul_fp8"
    return nd["dtype"] == head["dtype"]


def match_candidates(graph: Sequence[dict]) -> List[List[int]]:
    """Every chain that matches the pattern library, as node lists in chain order."""
    cons = consumers(graph)
    found: List[List[int]] = []
    for c, nd in enumerate(graph):
        if nd["op"] not in CONTRACTIONS:
            continue
        chain = [c]
        while True:
            last = chain[-1]
            # the value flowing on must have exactly one reader and must not be a graph
            # output, else fusing would take it from its other readers ([OPPL] §4.1, §4.2)
            if graph[last].get("output", False) or len(cons[last]) != 1:
                break
            nxt = cons[last][0]
            if not _step_ok(graph, chain, nxt):
                break
            chain = chain + [nxt]
            found.append(list(chain))
    return found


# ---- stage 2: benefit estimation -----------------------------------------------------------

def benefit(graph: Sequence[dict], chain: Sequence[int], ridge: float = DEFAULT_RIDGE,
            overhead_frac: float = DEFAULT_OVERHEAD_FRAC):
    """HBM bytes saved and net benefit of fusing the chain.

    Unfused, every op writes its output and the next op reads it back; fused, the first op
    reads the external inputs and only the last op writes.  The external reads (activations,
    residual, weights, per-channel vectors) are the same on both sides, so the saving is one
    write plus one read of every tensor inside the chain.  The overhead of the bigger kernel
    is a fixed fraction of the group's arithmetic, turned into bytes at the chip's
    flop-per-byte ratio.  Returns (saved_bytes, net); net is computed in binary64 as
    float(saved) - overhead_frac * float(flops) / ridge."""
    saved = 0
    for t in chain[:-1]:
        saved += 2 * tensor_bytes(graph[t])
    flops = 0
    for t in chain:
        flops += int(graph[t]["flops"])
    net = float(saved) - overhead_frac * float(flops) / ridge
    return saved, net


# ---- stage 3: conflict resolution -----------------------------------------------------------

def resolve_conflicts(cands: Sequence[dict]) -> List[dict]:
    """Greedy: candidates by net benefit, largest first; a candidate that shares an op with
    one already taken is dropped.  Each candidate is a dict with "nodes" and "net"; ties go
    to the chain that starts at the lower node index, then to the longer chain."""
    order = sorted(cands, key=lambda c: (-c["net"], c["nodes"][0], -len(c["nodes"])))
    taken = set()
    result = []
    for c in order:
        if any(op in taken for op in c["nodes"]):
            continue
        result.append(c)
        taken.update(c["nodes"])
    return result


def plan(graph: Sequence[dict], ridge: float = DEFAULT_RIDGE,
         overhead_frac: float = DEFAULT_OVERHEAD_FRAC) -> List[Dict]:
    """The three stages in order.  Returns the chosen groups, sorted by their first node:
    dicts with "nodes" (chain order), "saved" (bytes) and "net"."""
    cands = []
    for chain in match_candidates(graph):
        saved, net = benefit(graph, chain, ridge, overhead_frac)
        if net > 0:
            cands.append({"nodes": chain, "saved": saved, "net": net})
    groups = resolve_conflicts(cands)
    return sorted(groups, key=lambda g: g["nodes"][0])
