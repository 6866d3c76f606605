"""The library's host fusion pass (dlf_fusion_plan) against the pinned oracle pass, CPU only.

The plan is index work, so the bar is exact: the same groups, in the same order, with the
same saved bytes and bit-identical net benefits (both sides evaluate the benefit in binary64
in the same order of operations)."""
import ctypes

import pytest

from oracle import fusion
from workloads import graphs

dlf = pytest.importorskip("dl_fusion_amd", reason="libdlfusion.so not built")

RIDGE = fusion.DEFAULT_RIDGE
FRAC = fusion.DEFAULT_OVERHEAD_FRAC


def _same(graph, ridge=RIDGE, frac=FRAC):
    want = fusion.plan(graph, ridge, frac)
    got = dlf.dlf_fusion_plan(graph, ridge, frac)
    assert [g["nodes"] for g in got] == [g["nodes"] for g in want]
    assert [g["saved"] for g in got] == [g["saved"] for g in want]
    assert [g["net"].hex() for g in got] == [g["net"].hex() for g in want]
    return got


@pytest.mark.parametrize("seed", range(400))
def test_random_graphs_match_the_oracle(seed):
    _same(graphs.random_graph(seed, n_nodes=24))


@pytest.mark.parametrize("ridge,frac", [(RIDGE, FRAC), (RIDGE, 0.0), (10.0, 0.5), (1e4, 1.0)])
def test_overhead_parameters(ridge, frac):
    for seed in range(60):
        _same(graphs.random_graph(10_000 + seed, n_nodes=24), ridge, frac)


def test_network_graphs():
    g = graphs.resnet_stage_graph(n=32, h=56, w=56, cin=256, cmid=128, cout=512, stride=2, blocks=3)
    got = _same(g)
    assert [7, 8, 11, 12] in [p["nodes"] for p in got]
    assert [p["nodes"] for p in _same(graphs.stem_graph())] == [[1, 2, 3]]
    assert _same([]) == []


def _nodes(graph):
    return dlf.graph_nodes(graph)


def _plan_raw(arr, n, ridge=RIDGE, frac=FRAC, cap=8):
    out = (dlf.dlf_fusion_group * max(cap, 1))()
    cnt = ctypes.c_int32(-7)
    st = dlf.raw().dlf_fusion_plan(arr, n, ridge, frac, out if cap else None, cap, ctypes.byref(cnt))
    return st, cnt.value, out


def test_validation():
    g = graphs.resnet_stage_graph(n=2, h=8, w=8, cin=16, cmid=8, cout=32, stride=2, blocks=1)
    arr = _nodes(g)
    n = len(g)
    st, cnt, out = _plan_raw(arr, n)
    assert st == dlf.DLF_OK and cnt == 4
    # too small a capacity: the count needed comes back, nothing is written
    st, cnt, out = _plan_raw(arr, n, cap=2)
    assert st == dlf.DLF_ERR_INVALID_ARG and cnt == 4 and out[0].count == 0
    st, cnt, _ = _plan_raw(arr, n, cap=0)
    assert st == dlf.DLF_ERR_INVALID_ARG and cnt == 4
    for ridge, frac in ((0.0, FRAC), (float("inf"), FRAC), (RIDGE, -1.0), (RIDGE, float("nan"))):
        assert _plan_raw(arr, n, ridge, frac)[0] == dlf.DLF_ERR_INVALID_ARG
    bad = _nodes(g)
    bad[3].inputs[0] = 3                        # reads itself
    assert _plan_raw(bad, n)[0] == dlf.DLF_ERR_INVALID_ARG
    bad = _nodes(g)
    bad[2].op = 99
    assert _plan_raw(bad, n)[0] == dlf.DLF_ERR_INVALID_ARG
    bad = _nodes(g)
    bad[2].shape[1] = -1
    assert _plan_raw(bad, n)[0] == dlf.DLF_ERR_INVALID_ARG
    bad = _nodes(g)
    bad[2].rank = 5
    assert _plan_raw(bad, n)[0] == dlf.DLF_ERR_INVALID_ARG
    bad = _nodes(g)
    bad[1].flops = -1
    assert _plan_raw(bad, n)[0] == dlf.DLF_ERR_INVALID_ARG
    assert dlf.raw().dlf_fusion_plan(None, 3, RIDGE, FRAC, None, 0, ctypes.byref(ctypes.c_int32())) \
        == dlf.DLF_ERR_INVALID_ARG
    assert dlf.raw().dlf_fusion_plan(arr, n, RIDGE, FRAC, None, 0, None) == dlf.DLF_ERR_INVALID_ARG


def test_network_runner_plan_and_launches_on_the_host():
    """The runner's load-time work (plan, fold, buffers) without a GPU: the plan is the
    library's, one launch per chosen chain plus one per op outside a chain, and buffers only
    for the tensors the plan keeps in memory."""
    torch = pytest.importorskip("torch")
    from dl_fusion_amd.network import Network, OVERHEAD_FRAC, RIDGE_BF16
    g = graphs.resnet_stage_graph(n=2, h=8, w=8, cin=16, cmid=8, cout=32, stride=2, blocks=2)
    params = graphs.draw_params(g, seed=3)
    net = Network(g, params, fuse=True, device="cpu")
    plan = fusion.plan(g, RIDGE_BF16, OVERHEAD_FRAC)
    assert [p["nodes"] for p in net.plan] == [p["nodes"] for p in plan]
    inside = {i for p in plan for i in p["nodes"]}
    loose = [i for i, nd in enumerate(g) if nd["op"] != "input" and i not in inside]
    assert net.launches == len(plan) + len(loose)
    assert sorted(net.bufs) == sorted([p["nodes"][-1] for p in plan] + loose)
    assert net.saved_bytes == sum(p["saved"] for p in plan)
    plain = Network(g, params, fuse=False, device="cpu")
    assert plain.launches == sum(1 for nd in g if nd["op"] != "input") and plain.plan == []
    # what the runner refuses
    bad = [dict(nd) for nd in g]
    bad[2] = dict(bad[2], training=True)
    with pytest.raises(NotImplementedError):
        Network(bad, params, device="cpu")
    bad = [dict(nd) for nd in g]
    bad[1] = dict(bad[1], dtype="f32")
    with pytest.raises(NotImplementedError):
        Network(bad, params, device="cpu")
