"""Caller-side fallback on DLF_ERR_UNSUPPORTED (CPU only: host logic, no kernel runs).

A layer or a network chain whose fused call the library answers with DLF_ERR_UNSUPPORTED runs
its unfused chain instead ("OpenPPL算子融合深度解析" §4.2; the MindIE-SD RFC §3.7 falls back to
the original graph), and any other status is raised.  The statuses come from the library's own
host-side checks where a real unsupported shape exists (an FFN d_model the fused kernel is not
built for); elsewhere the fused entry point is replaced by one that answers UNSUPPORTED.  The
device calls of the unfused chain are replaced by recorders, and every tensor lives in host
memory, so nothing touches a GPU.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
dlf = pytest.importorskip("dl_fusion_amd")

import workloads  # noqa: E402
from dl_fusion_amd import layers, network  # noqa: E402


class Recorder:
    def __init__(self):
        self.calls = []

    def make(self, name):
        def fn(*args, **kw):
            self.calls.append((name, args))
        return fn


def unsupported(name):
    def fn(*args, **kw):
        raise dlf.DlfError(dlf.DLF_ERR_UNSUPPORTED, name)
    return fn


def failing(name, status):
    def fn(*args, **kw):
        raise dlf.DlfError(status, name)
    return fn


def test_ffn_unsupported_d_model_runs_two_gemms(monkeypatch):
    # d_model 384 has no fused kernel: the library's own check says UNSUPPORTED
    wl = workloads.FfnWorkload("ffn_384", m=40, d_model=384, d_ff=768, act="gelu_tanh", residual=True, seed=3)
    inp = workloads.generate(wl)
    with pytest.raises(dlf.DlfError) as e:
        dlf.dlf_ffn_workspace_bytes(dlf.ffn_desc(wl.m, wl.d_model, wl.d_ff, wl.act))
    assert e.value.status == dlf.DLF_ERR_UNSUPPORTED
    rec = Recorder()
    monkeypatch.setattr(layers, "dlf_gemm_fused", rec.make("gemm"))
    monkeypatch.setattr(layers, "dlf_ffn_fused_ws", failing("dlf_ffn_fused_ws", dlf.DLF_ERR_HIP))
    L = layers.make_layer(inp, device="cpu", with_unfused=False)
    assert not L.fused_ok and "d_model" in L.unsupported
    y = torch.empty((wl.m, wl.d_model), dtype=torch.bfloat16)
    assert L.forward(y=y) is y
    assert [c[0] for c in rec.calls] == ["gemm", "gemm"]
    (_, a1), (_, a2) = rec.calls
    assert a1[1] is L.x and a1[2] is L.w1 and a1[4] is L.b1 and a1[6] is L.h       # FC1 + b1 + act -> h
    assert a2[1] is L.h and a2[2] is L.w2 and a2[4] is L.b2 and a2[5] is L.res and a2[6] is y
    assert a1[0].act == dlf.ACTS["gelu_tanh"] and a2[0].act == dlf.ACTS["none"]


def test_conv_layer_falls_back_once_and_for_good(monkeypatch):
    wl = workloads.workload(2, n=1, h=4, w=4, cin=8, cout=16)
    inp = workloads.generate(wl)
    rec = Recorder()
    monkeypatch.setattr(layers, "dlf_conv_fused", unsupported("dlf_conv_fused"))
    for name in ("dlf_conv_plain", "dlf_bn_apply", "dlf_add", "dlf_act_apply"):
        monkeypatch.setattr(layers, name, rec.make(name))
    L = layers.make_layer(inp, device="cpu", with_unfused=False)
    y = L.forward()
    assert y is L.y and not L.fused_ok
    assert [c[0] for c in rec.calls] == ["dlf_conv_plain", "dlf_bn_apply", "dlf_add", "dlf_act_apply"]
    assert rec.calls[-1][1][4] is L.y                          # the chain writes the layer's output
    assert rec.calls[2][1][3] is L.res                         # the residual rides in the add
    # later calls go straight to the chain: the fused entry point is not asked again
    monkeypatch.setattr(layers, "dlf_conv_fused", failing("dlf_conv_fused", dlf.DLF_ERR_HIP))
    rec.calls.clear()
    L.forward()
    assert [c[0] for c in rec.calls] == ["dlf_conv_plain", "dlf_bn_apply", "dlf_add", "dlf_act_apply"]


@pytest.mark.parametrize("status", [dlf.DLF_ERR_INVALID_ARG, dlf.DLF_ERR_HIP, dlf.DLF_ERR_ALIAS])
def test_other_statuses_are_raised(monkeypatch, status):
    wl = workloads.workload(1, n=1, h=4, w=4)
    inp = workloads.generate(wl)
    rec = Recorder()
    monkeypatch.setattr(layers, "dlf_conv_fused", failing("dlf_conv_fused", status))
    monkeypatch.setattr(layers, "dlf_conv_plain", rec.make("dlf_conv_plain"))
    L = layers.make_layer(inp, device="cpu", with_unfused=False)
    with pytest.raises(dlf.DlfError) as e:
        L.forward()
    assert e.value.status == status and L.fused_ok and not rec.calls


def test_gemm_and_fp8_layers_fall_back(monkeypatch):
    rec = Recorder()
    monkeypatch.setattr(layers, "dlf_gemm_fused", unsupported("dlf_gemm_fused"))
    for name in ("dlf_gemm_plain", "dlf_scale_shift_apply", "dlf_add", "dlf_act_apply", "dlf_bn_apply",
                 "dlf_quant_apply"):
        monkeypatch.setattr(layers, name, rec.make(name))
    L = layers.make_layer(workloads.generate(workloads.workload(3, m=8, n=16, k=32)), device="cpu",
                          with_unfused=False)
    res = torch.empty((8, 16), dtype=torch.bfloat16)
    L.forward(residual=res)
    assert [c[0] for c in rec.calls] == ["dlf_gemm_plain", "dlf_scale_shift_apply", "dlf_add", "dlf_act_apply"]
    assert rec.calls[2][1][3] is res and rec.calls[-1][1][4] is L.y
    rec.calls.clear()
    L8 = layers.make_layer(workloads.generate(workloads.workload(4, m=8, n=16, k=32)), device="cpu",
                           with_unfused=False)
    L8.forward()
    assert [c[0] for c in rec.calls] == ["dlf_gemm_plain", "dlf_bn_apply", "dlf_act_apply", "dlf_quant_apply"]
    assert rec.calls[-1][1][3] is L8.y


def test_network_chain_runs_its_ops_when_unsupported(monkeypatch):
    from workloads import graphs
    g = graphs.resnet_stage_graph(n=1, h=8, w=8, cin=16, cmid=8, cout=32, stride=2, blocks=1)
    params = graphs.draw_params(g, seed=1)
    rec = Recorder()
    monkeypatch.setattr(network, "dlf_conv_fused", unsupported("dlf_conv_fused"))
    for name in ("dlf_conv_plain", "dlf_bn_apply", "dlf_add", "dlf_act_apply"):
        monkeypatch.setattr(network, name, rec.make(name))
    net = network.Network(g, params, fuse=True, device="cpu")
    assert net.plan
    x = {j: torch.empty(g[j]["shape"], dtype=torch.bfloat16) for j in net.inputs}
    net.forward(x)
    # every op of every chain ran on its own, in graph order, and each chain's last op wrote the
    # network's own buffer of the chain's result
    ops = [c[0] for c in rec.calls]
    expected = []
    for p in net.plan:
        for i in p["nodes"]:
            op = g[i]["op"]
            expected.append({"conv": "dlf_conv_plain", "batchnorm": "dlf_bn_apply", "add": "dlf_add"}.get(
                op, "dlf_act_apply"))
    assert sorted(ops) == sorted(expected) and len(ops) == len(expected)
    written = [c[1][-2] for c in rec.calls]
    for p in net.plan:
        assert any(t is net.bufs[p["nodes"][-1]] for t in written)
