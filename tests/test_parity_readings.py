"""Pins of the readings behind the parity metric and tolerances (CPU only).

Each test runs the method's own arithmetic exactly on the CPU - with the oracle's primitives,
never the HIP path - and shows that the bar the GPU tests apply is the one this arithmetic can
meet while the alternative reading cannot:

- R1, the per-channel floor of the relative error.  The method folds BN into the weights and
  rounds W' once to bf16 ("OpenPPL算子融合深度解析" §3.1, §6.2).  A channel whose BN scale
  gamma/sqrt(var + eps) is ten times the others' carries ten times their weight-rounding error,
  so a floor taken over the whole tensor judges it against the magnitude of the other channels.
  An exact implementation of the method (binary64 sums over the bf16 W', fp32 b', one bf16
  output rounding) misses 2e-2 under the tensor-wide floor and meets it with room under the
  per-channel floor, on both bf16 conv workloads.
- R2, the unfused chain's 4e-2.  The chain stores the conv output, the BN output and the
  residual sum as bf16 tensors, which the fused kernel keeps in fp32 registers ("OpenPPL算子融合
  深度解析" §2.1: every elementwise op writes its tensor back).  Exact arithmetic with only those
  storage roundings already exceeds 2e-2 on the residual workload, and stays inside 4e-2.
- R17, the pre-activation floor of a network step.  In a network whose BN statistics do not
  centre each channel's conv output (random running statistics over post-ReLU inputs), ReLU
  leaves some channels nearly empty: their rms after the activation is far below the size of
  the values the method rounded.  The exact method misses 2e-2 there under the per-channel
  floor of the output, and meets it with room under the per-channel floor of the value before
  the activation, on every fused step of a ResNet stage.
- R15, the row floor for fewer than 8 tokens.  With one or two tokens a column's rms is the
  element itself, so an output whose FC2 sum nearly cancels is judged on its own rounding:
  the exact FFN arithmetic (bf16 intermediate, bf16 output) fails the per-column floor there
  and meets the row floor; from a few dozen tokens on, the per-column floor holds.
"""
import numpy as np

import oracle
import workloads

BF16_TOL = 2e-2


def tensor_floor_error(got, ref) -> float:
    """max |g - o| / max(|o|, rms(o)), the rms taken over the whole tensor (the alternative
    reading of the floor that R1 rejects)."""
    g = np.asarray(got, dtype=np.float64)
    o = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(o * o))
    return float(np.max(np.abs(g - o) / np.maximum(np.abs(o), rms)))


def method_conv_exact(inp):
    """The fused operator's arithmetic with exact sums: fold in binary64, W' rounded once to
    bf16, b' stored as fp32, conv + b' [+ residual] -> activation, one bf16 output rounding."""
    wl = inp["workload"]
    w_f, b_f = oracle.fold_bn(inp["w"], inp["conv_bias"], inp["gamma"], inp["beta"], inp["mean"],
                              inp["var"], inp["eps"])
    w_q = oracle.round_bf16(w_f)
    b_32 = b_f.astype(np.float32)
    y = oracle.conv2d(oracle.widen(inp["x"], wl.dtype), w_q, b_32, wl.stride, wl.pad)
    if inp.get("residual") is not None:
        y = oracle.add(y, oracle.widen(inp["residual"], wl.dtype))
    return oracle.round_bf16(oracle.activation(y, wl.act))


def test_r1_channel_floor_is_the_one_the_method_meets():
    for idx, n in ((1, 4), (2, 8)):
        wl = workloads.workload(idx, n=n)
        inp = workloads.generate(wl)
        ref = oracle.conv_bn_act(inp)
        got = method_conv_exact(inp)
        per_channel = oracle.rel_error(got, ref)
        tensor_wide = tensor_floor_error(got, ref)
        assert tensor_wide > BF16_TOL, (idx, tensor_wide)
        assert per_channel < 0.75 * BF16_TOL, (idx, per_channel)


def test_r1_channel_scales_differ_by_more_than_ten():
    """The premise of R1 on the workloads themselves: the BN scales of one layer span more than a
    factor of ten (on the stressed-variance workload eps = 1e-2 caps the largest scales)."""
    for idx, span in ((1, 10.0), (2, 10.0)):
        inp = workloads.generate(workloads.workload(idx, n=1))
        s = inp["gamma"].astype(np.float64) / np.sqrt(inp["var"].astype(np.float64) + inp["eps"])
        assert s.max() / s.min() > span, (idx, s.max() / s.min())


def test_r2_unfused_chain_storage_roundings_exceed_the_fused_bar():
    wl = workloads.workload(2)
    inp = workloads.generate(wl)
    ref = oracle.conv_bn_act(inp)
    x = oracle.widen(inp["x"], wl.dtype)
    w = oracle.round_bf16(np.asarray(inp["w"], dtype=np.float64))      # bf16 master weights
    y = oracle.round_bf16(oracle.conv2d(x, w, inp["conv_bias"], wl.stride, wl.pad))
    z = oracle.round_bf16(oracle.batchnorm(y, inp["gamma"], inp["beta"], inp["mean"], inp["var"], inp["eps"]))
    u = oracle.round_bf16(oracle.add(z, oracle.widen(inp["residual"], wl.dtype)))
    out = oracle.round_bf16(oracle.relu(u))
    err = oracle.rel_error(out, ref)
    assert BF16_TOL < err < 0.8 * 4e-2, err
    # the fused arithmetic on the same inputs stays inside the fused bar
    assert oracle.rel_error(method_conv_exact(inp), ref) < 0.75 * BF16_TOL


def method_ffn_exact(inp):
    """The fused FFN's arithmetic with exact sums: h rounded to bf16 on chip, y rounded once."""
    wl = inp["workload"]
    x = oracle.widen(inp["x"], "bf16")
    h = oracle.activation(oracle.bias_add(oracle.matmul_nt(x, oracle.widen(inp["w1"], "bf16")), inp["b1"]), wl.act)
    y = oracle.bias_add(oracle.matmul_nt(oracle.round_bf16(h), oracle.widen(inp["w2"], "bf16")), inp["b2"])
    if inp.get("residual") is not None:
        y = oracle.add(y, oracle.widen(inp["residual"], "bf16"))
    return oracle.round_bf16(y)


def row_floor_error(got, ref) -> float:
    return oracle.rel_error(np.asarray(got).reshape(-1), np.asarray(ref).reshape(-1))


def test_r15_few_tokens_need_the_row_floor():
    for i, kw in enumerate([dict(m=1, d_model=256, d_ff=256, act="relu", residual=False),
                            dict(m=2, d_model=768, d_ff=3072, act="gelu_tanh", residual=False)]):
        wl = workloads.FfnWorkload(f"ffn_r15_{i}", seed=51 + i, **kw)
        inp = workloads.generate(wl)
        ref = oracle.ffn(inp)
        got = method_ffn_exact(inp)
        assert oracle.rel_error(got, ref) > BF16_TOL, i
        assert row_floor_error(got, ref) < 0.5 * BF16_TOL, i


def test_r15_column_floor_holds_from_a_few_dozen_tokens():
    for i, kw in enumerate([dict(m=37, d_model=768, d_ff=3072, act="gelu_tanh", residual=True),
                            dict(m=64, d_model=512, d_ff=1024, act="relu", residual=False)]):
        wl = workloads.FfnWorkload(f"ffn_r15b_{i}", seed=54 + i, **kw)
        inp = workloads.generate(wl)
        assert oracle.rel_error(method_ffn_exact(inp), oracle.ffn(inp)) < 0.75 * BF16_TOL, i


def test_r17_network_steps_need_the_pre_activation_floor():
    from oracle import fusion as ofusion, network as onet
    from workloads import graphs
    g = graphs.resnet_stage_graph(n=1, h=56, w=56, cin=256, cmid=128, cout=512, stride=2, blocks=2)
    params = graphs.draw_params(g, seed=7)
    plan = ofusion.plan(g, 2516.6e12 / 8.0e12, 0.05)
    bits = {j: workloads.bf16_bits(params[j]["x"]) for j, nd in enumerate(g) if nd["op"] == "input"}
    vals = onet.forward(g, params, bits, plan)
    worst_out, worst_pre = 0.0, 0.0
    for j, nodes in onet.steps(g, plan).items():
        c = nodes[0]
        if g[c]["op"] != "conv":
            continue
        pre, ref = onet.step(g, params, vals, nodes, with_pre=True)
        # the method's arithmetic for this step: fold, W' rounded once to bf16, exact sums
        bn, a = nodes[1], g[c]["attrs"]
        p = params[bn]
        w_f, b_f = oracle.fold_bn(params[c]["w"], None, p["gamma"], p["beta"], p["mean"], p["var"],
                                  g[bn]["attrs"]["eps"])
        y = oracle.conv2d(vals[g[c]["inputs"][0]], oracle.round_bf16(w_f), b_f.astype(np.float32), a["stride"],
                          a["pad"])
        prev = bn
        for i in nodes[2:]:
            if g[i]["op"] == "add":
                y = oracle.add(y, vals[[q for q in g[i]["inputs"] if q != prev][0]])
            else:
                y = oracle.activation(y, {"relu": "relu", "gelu": "gelu_tanh"}[g[i]["op"]])
            prev = i
        got = oracle.round_bf16(y)
        worst_out = max(worst_out, oracle.rel_error(got, ref))
        worst_pre = max(worst_pre, oracle.rel_error(got, ref, floor_of=pre))
    assert worst_out > BF16_TOL, worst_out
    assert worst_pre < 0.75 * BF16_TOL, worst_pre
