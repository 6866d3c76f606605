"""Pins of the fusion-pass oracle (oracle/fusion.py), CPU only.

Each stage is pinned to something other than itself: the worked example the CANN
graph-autofusion page prints for conflict resolution, its MatMul -> BiasAdd -> ReLU and
MatMul -> Reshape -> MatMul examples, the legality rules of [OPPL] §4.1-§4.2 on hand-built
graphs, a hand-traced ResNet stage, an independent regular-expression matcher for stage 1
and a brute-force set packing for stage 3.
"""
from __future__ import annotations

import itertools
import re

import numpy as np
import pytest

import oracle
from oracle import fusion
from workloads import graphs

MB = 1 << 20


def node(op, inputs, shape=(8, 16), dtype="bf16", flops=0, output=False, training=False):
    return dict(op=op, inputs=list(inputs), shape=tuple(shape), dtype=dtype, flops=flops,
                output=output, training=training)


def test_conflict_example_of_the_autofusion_page():
    """[CANN] stage 3: on A -> B -> C -> D, group {A, B, C} saves 120 MB and {B, C, D} 100 MB;
    they share B and C, so the larger one is taken and the other dropped."""
    cands = [{"nodes": ["B", "C", "D"], "net": 100.0 * MB},
             {"nodes": ["A", "B", "C"], "net": 120.0 * MB}]
    got = fusion.resolve_conflicts(cands)
    assert [g["nodes"] for g in got] == [["A", "B", "C"]]
    # disjoint candidates are both taken, largest first
    got = fusion.resolve_conflicts([{"nodes": ["A"], "net": 1.0}, {"nodes": ["B"], "net": 2.0}])
    assert [g["nodes"] for g in got] == [["B"], ["A"]]


def test_matmul_bias_relu_saves_two_round_trips():
    """[CANN]: MatMul -> BiasAdd -> ReLU goes from three HBM round trips to one.  The two
    tensors between the ops are neither written nor read back."""
    m, n = 64, 96
    g = [node("input", [], (m, 32)),
         node("matmul", [0], (m, n), flops=2 * m * n * 32),
         node("bias_add", [1], (m, n), flops=m * n),
         node("relu", [2], (m, n), flops=m * n, output=True)]
    assert fusion.match_candidates(g) == [[1, 2], [1, 2, 3]]
    saved, net = fusion.benefit(g, [1, 2, 3])
    assert saved == 2 * 2 * (m * n * 2)              # two intermediates, written and read once each
    plan = fusion.plan(g)
    assert [p["nodes"] for p in plan] == [[1, 2, 3]]
    assert plan[0]["saved"] == saved


def test_matmul_reshape_matmul_is_no_candidate():
    """[CANN]: a Reshape between two MatMuls saves nothing; it belongs to no pattern."""
    g = [node("input", [], (8, 16)),
         node("matmul", [0], (8, 32), flops=4096),
         node("reshape", [1], (16, 16)),
         node("matmul", [2], (16, 8), flops=4096, output=True)]
    assert fusion.match_candidates(g) == []
    assert fusion.plan(g) == []


def test_unique_consumer_training_bn_and_broadcast():
    """[OPPL] §4.1-§4.2: a conv output read twice, a BN in training mode, an intermediate that
    is a graph output and an Add whose other operand has another shape all stop the chain."""
    # conv read by the BN and by a second branch: nothing fuses behind the conv
    g = [node("input", []), node("conv", [0], flops=100), node("batchnorm", [1]), node("relu", [2]),
         node("relu", [1], output=True)]
    assert fusion.match_candidates(g) == []
    # BN in training mode
    g = [node("input", []), node("conv", [0], flops=100), node("batchnorm", [1], training=True),
         node("relu", [2], output=True)]
    assert fusion.match_candidates(g) == []
    # the BN output is itself a graph output: conv + BN may fuse, the ReLU may not join
    g = [node("input", []), node("conv", [0], flops=100), node("batchnorm", [1], output=True),
         node("relu", [2], output=True)]
    assert fusion.match_candidates(g) == [[1, 2]]
    # residual of another shape (a broadcast) or another dtype
    for other in (node("input", [], (1, 16)), node("input", [], (8, 16), dtype="f32")):
        g = [node("input", []), other, node("conv", [0], flops=100), node("batchnorm", [2]),
             node("add", [3, 1]), node("relu", [4], output=True)]
        assert fusion.match_candidates(g) == [[2, 3]]
    # same-shape residual: the whole chain, in either operand slot
    for slots in ([3, 1], [1, 3]):
        g = [node("input", []), node("input", []), node("conv", [0], flops=100), node("batchnorm", [2]),
             node("add", slots), node("relu", [4], output=True)]
        assert fusion.match_candidates(g) == [[2, 3], [2, 3, 4], [2, 3, 4, 5]]
    # the epilogue order is fixed: an activation before the BN ends the chain
    g = [node("input", []), node("conv", [0], flops=100), node("relu", [1]), node("batchnorm", [2]),
         node("relu", [3], output=True)]
    assert fusion.match_candidates(g) == [[1, 2]]
    # quantisation closes only the fp8 MatMul's chain, which takes no residual
    g = [node("input", [], dtype="fp8"), node("matmul_fp8", [0], dtype="f32", flops=100),
         node("batchnorm", [1], dtype="f32"), node("relu", [2], dtype="f32"),
         node("quant", [3], dtype="fp8", output=True)]
    assert fusion.match_candidates(g) == [[1, 2], [1, 2, 3], [1, 2, 3, 4]]
    g[1]["op"] = "matmul"
    assert fusion.match_candidates(g) == [[1, 2], [1, 2, 3]]


def test_resnet_stage_hand_traced():
    """A two-block bottleneck stage (bf16, N=32, 56x56x256 -> 28x28x512).  The first block's
    main branch (1x1 conv over 128 channels) and its downsample branch (strided 1x1 over 256)
    both match Conv -> BN -> Add -> ReLU; they save the same bytes, the main branch's conv has
    half the arithmetic and so the smaller overhead, so it takes the Add and the downsample
    branch keeps Conv -> BN."""
    g = graphs.resnet_stage_graph(n=32, h=56, w=56, cin=256, cmid=128, cout=512, stride=2, blocks=2)
    ops = [nd["op"] for nd in g]
    assert ops[7:13] == ["conv", "batchnorm", "conv", "batchnorm", "add", "relu"]
    plan = fusion.plan(g)
    assert [p["nodes"] for p in plan] == [[1, 2, 3], [4, 5, 6], [7, 8, 11, 12], [9, 10], [13, 14, 15],
                                          [16, 17, 18], [19, 20, 21, 22]]
    t28 = 32 * 28 * 28 * 512 * 2
    assert plan[2]["saved"] == 3 * 2 * t28
    assert plan[3]["saved"] == 1 * 2 * t28
    t56 = 32 * 56 * 56 * 128 * 2
    assert plan[0]["saved"] == 2 * 2 * t56
    f_main = 2 * 32 * 28 * 28 * 512 * 128 + (2 + 1 + 1) * (32 * 28 * 28 * 512)   # conv, BN, add, ReLU
    assert plan[2]["net"] == float(3 * 2 * t28) - 0.05 * float(f_main) / fusion.DEFAULT_RIDGE


# ---- stage 1 against a regular expression over paths ---------------------------------------

_PATTERN = re.compile(r"^(conv|matmul|matmul_fp8)( (bias_add|batchnorm))?( add)?( (relu|gelu|gelu_erf))?( quant)?$")


def _brute_candidates(g):
    """All paths head -> ... along producer/consumer edges, written as op strings and kept when
    the regular expression accepts them and every local rule holds."""
    cons = [[i for i, nd in enumerate(g) for j in nd["inputs"] if j == p] for p in range(len(g))]
    out = []

    def ok(path):
        head = g[path[0]]
        for a, b in zip(path, path[1:]):
            if g[a].get("output") or cons[a] != [b]:
                return False
        for b in path[1:]:
            nd = g[b]
            if tuple(nd["shape"]) != tuple(head["shape"]):
                return False
            if nd["op"] == "batchnorm" and nd["training"]:
                return False
            if nd["op"] == "quant":
                if head["op"] != "matmul_fp8" or len(nd["inputs"]) != 1:
                    return False
            elif nd["op"] == "add":
                prev = path[path.index(b) - 1]
                if head["op"] == "matmul_fp8" or sorted(nd["inputs"]).count(prev) != 1 or len(nd["inputs"]) != 2:
                    return False
                r = g[[j for j in nd["inputs"] if j != prev][0]]
                if tuple(r["shape"]) != tuple(nd["shape"]) or r["dtype"] != nd["dtype"] or nd["dtype"] != head["dtype"]:
                    return False
            else:
                if len(nd["inputs"]) != 1 or nd["dtype"] != head["dtype"]:
                    return False
        return True

    def walk(path):
        if len(path) >= 2 and _PATTERN.match(" ".join(g[i]["op"] for i in path)) and ok(path):
            out.append(list(path))
        if len(path) < 6:
            for c in set(cons[path[-1]]):
                walk(path + [c])

    for i, nd in enumerate(g):
        if nd["op"] in fusion.CONTRACTIONS:
            walk([i])
    return sorted(out)


@pytest.mark.parametrize("seed", range(300))
def test_stage1_matches_brute_force_paths(seed):
    g = graphs.random_graph(seed, n_nodes=24)
    assert sorted(fusion.match_candidates(g)) == _brute_candidates(g)


def test_random_graphs_reach_every_rule():
    """The random graphs exercise the pass: over the seeds above, chains of every length and
    every kind of epilogue op are matched."""
    seen_len, seen_ops = set(), set()
    for seed in range(300):
        g = graphs.random_graph(seed, n_nodes=24)
        for c in fusion.match_candidates(g):
            seen_len.add(len(c))
            seen_ops.update(g[i]["op"] for i in c)
    assert {2, 3, 4} <= seen_len
    assert {"bias_add", "batchnorm", "add", "relu", "quant"} <= seen_ops


# ---- stage 3 against brute-force set packing -------------------------------------------------

@pytest.mark.parametrize("seed", range(200))
def test_greedy_is_a_maximal_packing_below_the_optimum(seed):
    rng = np.random.default_rng(1000 + seed)
    ops = list(range(8))
    cands = []
    for _ in range(int(rng.integers(1, 8))):
        k = int(rng.integers(1, 4))
        start = int(rng.integers(0, 8 - k + 1))
        cands.append({"nodes": ops[start:start + k], "net": float(rng.integers(1, 6))})
    got = fusion.resolve_conflicts(cands)
    used = [op for c in got for op in c["nodes"]]
    assert len(used) == len(set(used))                             # disjoint
    for c in cands:                                                 # maximal
        assert c in got or any(op in used for op in c["nodes"])
    best = 0.0                                                      # exhaustive optimum
    for r in range(len(cands) + 1):
        for sub in itertools.combinations(cands, r):
            u = [op for c in sub for op in c["nodes"]]
            if len(u) == len(set(u)):
                best = max(best, sum(c["net"] for c in sub))
    total = sum(c["net"] for c in got)
    assert total <= best
    assert got[0]["net"] == max(c["net"] for c in cands)            # the largest goes first
    # on nested prefixes of one chain (what stage 1 emits for a single contraction) the
    # greedy choice is the optimum: the longest prefix
    chain = [{"nodes": ops[:k], "net": float(k)} for k in range(1, 5)]
    assert [c["nodes"] for c in fusion.resolve_conflicts(chain)] == [ops[:4]]


def test_net_benefit_threshold():
    """Stage 2 drops a candidate whose overhead eats the saving: a tiny chain over a huge
    contraction is not fused."""
    g = [node("input", [], (2, 2)), node("matmul", [0], (2, 2), flops=10 ** 12),
         node("relu", [1], (2, 2), output=True)]
    saved, net = fusion.benefit(g, [1, 2])
    assert saved == 16 and net < 0
    assert fusion.plan(g) == []
    assert [p["nodes"] for p in fusion.plan(g, overhead_frac=0.0)] == [[1, 2]]


# ---- the network oracle ----------------------------------------------------------------------

def _identity_block(n=2, h=5, w=6, c=8):
    g = [dict(op="input", inputs=[], shape=(n, h, w, c), dtype="bf16", flops=0, output=False, training=False,
              attrs={}),
         dict(op="conv", inputs=[0], shape=(n, h, w, c), dtype="bf16", flops=2 * n * h * w * c * c, output=False,
              training=False, attrs=dict(kh=1, kw=1, stride=1, pad=0, cin=c, cout=c)),
         dict(op="batchnorm", inputs=[1], shape=(n, h, w, c), dtype="bf16", flops=1, output=False, training=False,
              attrs=dict(eps=0.0)),
         dict(op="add", inputs=[2, 0], shape=(n, h, w, c), dtype="bf16", flops=1, output=False, training=False,
              attrs={}),
         dict(op="relu", inputs=[3], shape=(n, h, w, c), dtype="bf16", flops=1, output=True, training=False,
              attrs={})]
    params = {0: {"x": np.random.default_rng(3).standard_normal((n, h, w, c)).astype(np.float32)},
              1: {"w": np.eye(c, dtype=np.float32).reshape(c, 1, 1, c)},
              2: {"gamma": np.ones(c, np.float32), "beta": np.zeros(c, np.float32),
                  "mean": np.zeros(c, np.float32), "var": np.ones(c, np.float32)}}
    return g, params


def test_network_oracle_identity_block_is_exact():
    """A 1x1 identity conv, an identity BN (gamma 1, beta 0, mean 0, var 1, eps 0) and a
    residual of the block input: the block computes relu(2 x), exactly in bf16, fused or not."""
    from oracle import network as onet
    import workloads as W
    g, params = _identity_block()
    bits = W.bf16_bits(params[0]["x"])
    x = oracle.widen(bits, "bf16")
    plan = fusion.plan(g)
    assert [p["nodes"] for p in plan] == [[1, 2, 3, 4]]
    for pl in (plan, []):
        out = onet.forward(g, params, {0: bits}, pl)
        np.testing.assert_array_equal(out[4], np.maximum(2 * x, 0.0))
    # the fused network keeps only the input and the result in memory
    assert sorted(onet.forward(g, params, {0: bits}, plan)) == [0, 4]


def test_network_oracle_routes_a_resnet_stage_exactly():
    """Every conv a channel selection at its centre tap (OHWI delta, identity on the first
    min(cin, cout) channels), every BN the identity: the two-block stage then computes, in
    exact bf16 arithmetic (values double at most), out1 = relu(S(x', cout) + S(x', cout)) on
    the selected channels where x' = relu(x)[:, ::2, ::2] for the main branch and x[:, ::2, ::2]
    for the shortcut, and out2 = relu(2 * out1) on the first cmid channels, out1 elsewhere.
    Pins the oracle's routing (strides, padding, the shortcut operand, the residual slot),
    fused and unfused."""
    from oracle import network as onet
    import workloads as W
    n, h, w, cin, cmid, cout = 2, 8, 10, 16, 8, 24
    g = graphs.resnet_stage_graph(n=n, h=h, w=w, cin=cin, cmid=cmid, cout=cout, stride=2, blocks=2)
    params = graphs.draw_params(g, seed=4)
    for i, nd in enumerate(g):
        if nd["op"] == "conv":
            a = nd["attrs"]
            wt = np.zeros((a["cout"], a["kh"], a["kw"], a["cin"]), np.float32)
            for c in range(min(a["cin"], a["cout"])):
                wt[c, a["kh"] // 2, a["kw"] // 2, c] = 1.0
            params[i] = {"w": wt}
        elif nd["op"] == "batchnorm":
            c = nd["shape"][-1]
            nd["attrs"]["eps"] = 0.0
            params[i] = {"gamma": np.ones(c, np.float32), "beta": np.zeros(c, np.float32),
                         "mean": np.zeros(c, np.float32), "var": np.ones(c, np.float32)}
    bits = W.bf16_bits(params[0]["x"])
    x = oracle.widen(bits, "bf16")

    def sel(t, c):
        out = np.zeros(t.shape[:-1] + (c,))
        k = min(c, t.shape[-1])
        out[..., :k] = t[..., :k]
        return out

    xs = x[:, ::2, ::2, :]
    main = sel(sel(np.maximum(sel(x, cmid), 0)[:, ::2, ::2, :], cmid), cout)
    out1 = np.maximum(main + sel(xs, cout), 0)
    out2 = np.maximum(sel(sel(np.maximum(sel(out1, cmid), 0), cmid), cout) + out1, 0)
    for pl in (fusion.plan(g), []):
        got = onet.forward(g, params, {0: bits}, pl)
        np.testing.assert_array_equal(got[12], out1)
        np.testing.assert_array_equal(got[len(g) - 1], out2)
