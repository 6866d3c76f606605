"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks one oracle step against a closed form, an invariant, a
hand-worked example (tests/golden), brute force in an independent formulation,
or a library routine that computes the same textbook function.  The cases are
chosen so that a plausible slip (a dropped term, a swapped index, a wrong sign,
a missed epsilon, an off-by-one in the padding) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Independent formulations used only as pins
# ---------------------------------------------------------------------------
def im2col_conv(x, w, bias, stride, pad):
    """Convolution as im2col + a numpy float64 matmul (library routine), NHWC/OHWI."""
    n, h, wd, cin = x.shape
    cout, kh, kw, _ = w.shape
    xp = np.zeros((n, h + 2 * pad, wd + 2 * pad, cin))
    xp[:, pad:pad + h, pad:pad + wd, :] = x
    ho = (h + 2 * pad - kh) // stride + 1
    wo = (wd + 2 * pad - kw) // stride + 1
    cols = np.empty((n, ho, wo, kh, kw, cin))
    for r in range(kh):
        for s in range(kw):
            cols[:, :, :, r, s, :] = xp[:, r:r + stride * ho:stride, s:s + stride * wo:stride, :]
    y = cols.reshape(n * ho * wo, -1) @ w.reshape(cout, -1).T
    if bias is not None:
        y = y + bias
    return y.reshape(n, ho, wo, cout)


def e4m3_int(codes):
    """e4m3 magnitudes as exact integers in units of 2^-9 (sign applied), from the format's
    closed form: subnormal m -> m; normal (e, m) -> (8 + m) * 2^(e - 1)."""
    c = codes.astype(np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m, (8 + m) << np.maximum(e - 1, 0))
    return np.where(c & 0x80, -mag, mag)


# ---------------------------------------------------------------------------
# O2: convolution
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("k", [1, 3])
@pytest.mark.parametrize("stride", [1, 2])
@pytest.mark.parametrize("pad", [0, 1])
def test_conv_matches_im2col_brute_force(k, stride, pad):
    rng = np.random.default_rng(100 + 10 * k + 3 * stride + pad)
    for trial in range(4):
        n, h, w, cin, cout = rng.integers(1, 3), rng.integers(k, 6), rng.integers(k, 6), rng.integers(1, 4), rng.integers(1, 4)
        x = rng.standard_normal((n, h, w, cin))
        wt = rng.standard_normal((cout, k, k, cin))
        b = rng.standard_normal(cout) if trial % 2 else None
        got = oracle.conv2d(x, wt, b, stride, pad)
        ref = im2col_conv(x, wt, b, stride, pad)
        assert got.shape == ref.shape
        np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_conv_points_match_full_conv():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 7, 6, 5))
    wt = rng.standard_normal((4, 3, 3, 5))
    b = rng.standard_normal(4)
    full = oracle.conv2d(x, wt, b, 2, 1)
    pts = np.array([[0, 0, 0], [1, 3, 2], [0, 2, 1], [1, 0, 2]])
    got = oracle.conv2d_at(x, wt, pts, b, 2, 1)
    np.testing.assert_array_equal(got, full[pts[:, 0], pts[:, 1], pts[:, 2]])


def test_conv_1x1_is_matmul():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 4, 5, 6))
    wt = rng.standard_normal((3, 1, 1, 6))
    got = oracle.conv2d(x, wt, None, 1, 0)
    ref = (x.reshape(-1, 6) @ wt.reshape(3, 6).T).reshape(2, 4, 5, 3)
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(oracle.matmul_nt(x.reshape(-1, 6), wt.reshape(3, 6)), ref.reshape(-1, 3),
                               rtol=1e-14, atol=1e-14)


def test_conv_delta_kernel_is_identity():
    rng = np.random.default_rng(2)
    c = 3
    x = rng.standard_normal((2, 5, 4, c))
    wt = np.zeros((c, 3, 3, c))
    for i in range(c):
        wt[i, 1, 1, i] = 1.0
    np.testing.assert_array_equal(oracle.conv2d(x, wt, None, 1, 1), x)


@pytest.mark.parametrize("cin", [1, 3, 8])
def test_conv_all_ones_counts_in_bounds_taps(cin):
    """All-ones x and W: each output is cin * (number of taps inside the image):
    4 cin at corners, 6 cin on edges, 9 cin inside (pins the zero padding)."""
    h, w = 5, 6
    y = oracle.conv2d(np.ones((1, h, w, cin)), np.ones((2, 3, 3, cin)), None, 1, 1)
    rows = np.array([2] + [3] * (h - 2) + [2])
    cols = np.array([2] + [3] * (w - 2) + [2])
    expected = cin * np.outer(rows, cols)
    for co in range(2):
        np.testing.assert_array_equal(y[0, :, :, co], expected)
    assert y[0, 0, 0, 0] == 4 * cin and y[0, 0, 2, 0] == 6 * cin and y[0, 2, 2, 0] == 9 * cin


def test_conv_small_integers_exact_against_int64():
    rng = np.random.default_rng(3)
    x = rng.integers(-8, 9, (2, 6, 5, 4))
    wt = rng.integers(-8, 9, (3, 3, 3, 4))
    b = rng.integers(-50, 51, 3)
    got = oracle.conv2d(x.astype(np.float64), wt.astype(np.float64), b.astype(np.float64), 1, 1)
    xp = np.zeros((2, 8, 7, 4), dtype=np.int64)
    xp[:, 1:7, 1:6, :] = x
    ref = np.zeros((2, 6, 5, 3), dtype=np.int64)
    for r in range(3):
        for s in range(3):
            ref += np.einsum("nhwc,oc->nhwo", xp[:, r:r + 6, s:s + 5, :], wt[:, r, s, :])
    ref += b
    np.testing.assert_array_equal(got, ref.astype(np.float64))


def test_hand_worked_conv_bn_relu_golden():
    rows = np.loadtxt(os.path.join(GOLDEN, "conv_bn_relu_hand.txt"), comments="#")
    x = np.arange(1, 10, dtype=np.float64).reshape(1, 3, 3, 1)
    wt = np.stack([np.ones((3, 3, 1)), 2 * np.ones((3, 3, 1))])
    bias = np.array([1.0, 0.0])
    gamma, beta = np.array([2.0, 1.5]), np.array([-30.0, 0.5])
    mean, var, eps = np.array([1.0, 10.0]), np.array([3.0, 3.0]), 1.0
    y = oracle.conv2d(x, wt, bias, 1, 1)
    z = oracle.relu(oracle.batchnorm(y, gamma, beta, mean, var, eps))
    for ho, wo, y0, y1, z0, z1 in rows:
        ho, wo = int(ho), int(wo)
        assert y[0, ho, wo, 0] == y0 and y[0, ho, wo, 1] == y1
        assert z[0, ho, wo, 0] == z0 and z[0, ho, wo, 1] == z1
    w_f, b_f = oracle.fold_bn(wt, bias, gamma, beta, mean, var, eps)
    assert np.all(w_f[0] == 1.0) and np.all(w_f[1] == 1.5)
    assert b_f.tolist() == [-30.0, -7.0]
    zf = oracle.relu(oracle.conv2d(x, w_f, b_f, 1, 1))
    np.testing.assert_array_equal(zf, z)


# ---------------------------------------------------------------------------
# O3 / O9: BatchNorm and the fold
# ---------------------------------------------------------------------------
def test_batchnorm_matches_torch_inference_batch_norm():
    rng = np.random.default_rng(4)
    y = rng.standard_normal((37, 11))
    g, b = rng.uniform(0.5, 1.5, 11), rng.normal(0, 0.1, 11)
    mu, var = rng.normal(0, 0.1, 11), rng.uniform(1e-6, 1, 11)
    for eps in (1e-5, 1e-2, 1e-9):
        ref = torch.nn.functional.batch_norm(torch.from_numpy(y), torch.from_numpy(mu), torch.from_numpy(var),
                                             torch.from_numpy(g), torch.from_numpy(b), training=False, eps=eps)
        np.testing.assert_allclose(oracle.batchnorm(y, g, b, mu, var, eps), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_batchnorm_identity_and_shift_cases():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((9, 4))
    ones = np.ones(4)
    eps = 0.25
    var = np.full(4, 0.75)      # var + eps = 1 exactly
    np.testing.assert_array_equal(oracle.batchnorm(y, ones, np.zeros(4), np.zeros(4), var, eps), y)
    mu, beta = np.array([0.5, -1.0, 2.0, 0.0]), np.array([1.0, 0.25, -3.0, 4.0])
    np.testing.assert_allclose(oracle.batchnorm(y, ones, beta, mu, var, eps), y - mu + beta, rtol=0, atol=1e-15)
    # gamma = 2, var + eps = 4: scale exactly 1
    np.testing.assert_array_equal(oracle.batchnorm(y, 2 * ones, np.zeros(4), np.zeros(4), np.full(4, 3.75), eps), y)


@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("eps", [1e-5, 1e-2])
def test_fold_closed_form_folded_equals_unfolded(with_bias, eps):
    """Conv with (W', b') equals conv -> BN to 1e-12 (the fold is an identity)."""
    wl = workloads.workload(2, n=2, h=6, w=5, cin=16, cout=24, conv_bias=with_bias, eps=eps)
    inp = workloads.generate(wl)
    x = oracle.widen(inp["x"], "bf16")
    unfolded = oracle.batchnorm(oracle.conv2d(x, inp["w"], inp["conv_bias"]), inp["gamma"], inp["beta"],
                                inp["mean"], inp["var"], eps)
    w_f, b_f = oracle.fold_bn(inp["w"], inp["conv_bias"], inp["gamma"], inp["beta"], inp["mean"], inp["var"], eps)
    folded = oracle.conv2d(x, w_f, b_f)
    assert oracle.rel_error(folded, unfolded) <= 1e-12


def test_fold_without_bias_equals_fold_with_zero_bias():
    inp = workloads.generate(workloads.workload(1, n=1, h=4, w=4, cout=8, cin=8))
    a = oracle.fold_bn(inp["w"], None, inp["gamma"], inp["beta"], inp["mean"], inp["var"], 1e-5)
    b = oracle.fold_bn(inp["w"], np.zeros(8), inp["gamma"], inp["beta"], inp["mean"], inp["var"], 1e-5)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_negative_control_dropping_eps_fails_the_bf16_check():
    """With eps dropped (0 instead of the model's 1e-2), the stressed low-variance
    channels change by a large factor: the bf16 tolerance must reject it.  This shows
    the comparison is sensitive to eps handling."""
    inp = workloads.generate(workloads.workload(2, n=2, h=6, w=6))
    ok = oracle.conv_bn_act(inp)
    bad = oracle.conv_bn_act(inp, eps=0.0)
    assert oracle.rel_error(bad, ok) > 2e-2
    st = inp["stressed"]
    assert st.size == 26
    ratio = np.sqrt((inp["var"][st].astype(np.float64) + 1e-2) / inp["var"][st])
    assert ratio.min() > 3.0 and ratio.max() < 101.0


# ---------------------------------------------------------------------------
# O4 / O5: residual and activations
# ---------------------------------------------------------------------------
def test_residual_linearity_cancels_exactly():
    rng = np.random.default_rng(6)
    y = oracle.conv2d(rng.standard_normal((1, 5, 5, 3)), rng.standard_normal((4, 3, 3, 3)))
    z = oracle.add(y, -y)
    assert np.all(z == 0.0)
    assert np.all(oracle.relu(z) == 0.0)


def test_relu_invariants():
    rng = np.random.default_rng(7)
    u = np.concatenate([rng.standard_normal(1000), [0.0, -0.0, 1e-300, -1e-300]])
    r = oracle.relu(u)
    assert np.all(r >= 0)
    np.testing.assert_array_equal(r[u > 0], u[u > 0])
    assert np.all(r[u <= 0] == 0.0)
    assert not np.any(np.signbit(r))


def test_gelu_tanh_identities_and_library():
    rng = np.random.default_rng(8)
    u = np.concatenate([rng.standard_normal(2000) * 4, np.linspace(-10, 10, 201)])
    g, gm = oracle.gelu_tanh(u), oracle.gelu_tanh(-u)
    # tanh is odd => gelu(u) - gelu(-u) = u
    np.testing.assert_allclose(g - gm, u, rtol=1e-14, atol=1e-15)
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    ref = torch.nn.functional.gelu(torch.from_numpy(u), approximate="tanh").numpy()
    np.testing.assert_allclose(g, ref, rtol=1e-14, atol=1e-15)
    # large |u| limits: gelu -> u for u >> 0, -> 0 for u << 0
    assert oracle.gelu_tanh(np.array([30.0]))[0] == 30.0
    assert abs(oracle.gelu_tanh(np.array([-30.0]))[0]) < 1e-300


def test_gelu_erf_is_u_times_normal_cdf():
    """Exact GELU ([RFC] §2.1, §2.4) = u Phi(u): pinned to scipy's normal CDF, the odd symmetry
    of erf, a textbook value, and a measurable gap to the tanh form (which must not stand in)."""
    from scipy.stats import norm
    rng = np.random.default_rng(11)
    u = np.concatenate([rng.standard_normal(2000) * 4, np.linspace(-12, 12, 241)])
    g = oracle.gelu_erf(u)
    np.testing.assert_allclose(g, u * norm.cdf(u), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(g - oracle.gelu_erf(-u), u, rtol=1e-14, atol=1e-15)   # erf is odd
    assert oracle.gelu_erf(np.array([0.0]))[0] == 0.0
    assert abs(oracle.gelu_erf(np.array([1.0]))[0] - 0.8413447460685429) < 1e-15   # Phi(1)
    assert oracle.gelu_erf(np.array([40.0]))[0] == 40.0
    assert abs(oracle.gelu_erf(np.array([-40.0]))[0]) < 1e-300
    gap = np.abs(g - oracle.gelu_tanh(u))
    assert 1e-4 < gap.max() < 1e-3, gap.max()


def test_split_gemm_equals_separate_projections():
    """[OPPL] §3.2: one GEMM over [W_q; W_k; W_v] cut into three column blocks equals the three
    projections computed separately (here with numpy on the blocks, not the oracle's matmul)."""
    for act in ("none", "gelu_erf"):
        wl = workloads.workload(3, m=7, n=3 * 16, k=40, act=act, bias=True)
        inp = workloads.generate(wl)
        parts = oracle.gemm_bias_act_split(inp, 3)
        x = oracle.widen(inp["x"], "bf16")
        w = oracle.widen(inp["w"], "bf16")
        for p, got in enumerate(parts):
            sl = slice(16 * p, 16 * (p + 1))
            ref = x @ w[sl].T + inp["bias"][sl].astype(np.float64)
            if act == "gelu_erf":
                from scipy.stats import norm
                ref = ref * norm.cdf(ref)
            assert got.shape == (7, 16)
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.gemm_bias_act_split(inp, 5)


def test_silu_against_the_logistic_function():
    from scipy.special import expit
    rng = np.random.default_rng(12)
    u = np.concatenate([rng.standard_normal(2000) * 6, np.linspace(-30, 30, 121)])
    np.testing.assert_allclose(oracle.silu(u), u * expit(u), rtol=1e-14, atol=1e-300)
    # silu(u) - silu(-u) = u (the logistic function's symmetry); silu(0) = 0
    np.testing.assert_allclose(oracle.silu(u) - oracle.silu(-u), u, rtol=1e-13, atol=1e-13)
    assert oracle.silu(np.array([0.0]))[0] == 0.0


def test_gated_projection_matches_separate_gate_and_up():
    """One MatMul over interleaved [g0; u0; g1; u1; ...] rows = act(x Wg^T + bg) * (x Wu^T + bu),
    computed here with numpy on the de-interleaved weights and scipy's logistic / normal CDF."""
    from scipy.special import expit
    from scipy.stats import norm
    wl = workloads.workload(3, m=6, n=2 * 24, k=32, act="none", bias=True)
    inp = workloads.generate(wl)
    x, w = oracle.widen(inp["x"], "bf16"), oracle.widen(inp["w"], "bf16")
    b = inp["bias"].astype(np.float64)
    g = x @ w[0::2].T + b[0::2]
    u = x @ w[1::2].T + b[1::2]
    forms = {"silu": g * expit(g), "gelu_erf": g * norm.cdf(g),
             "gelu_tanh": 0.5 * g * (1 + np.tanh(np.sqrt(2 / np.pi) * (g + 0.044715 * g ** 3)))}
    for gate, ga in forms.items():
        got = oracle.gemm_gated(inp, gate)
        assert got.shape == (6, 24)
        np.testing.assert_allclose(got, ga * u, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# O6 / O7: the fp8 e4m3 codec and the exact fp8 product
# ---------------------------------------------------------------------------
def test_e4m3_golden_points():
    with open(os.path.join(GOLDEN, "e4m3_ocp_points.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            code_s, val_s = line.split()
            code, val = int(code_s, 16), float(val_s)
            got = oracle.e4m3_value(code)
            if math.isnan(val):
                assert math.isnan(got)
                continue
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (code_s, got, val)
            assert oracle.e4m3_encode(np.array([val]))[0] == code


def test_e4m3_round_trip_and_monotone():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert codes.size == 254
    vals = oracle.e4m3_decode(codes)
    np.testing.assert_array_equal(oracle.e4m3_encode(vals), codes)
    pos = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0


def test_e4m3_ties_go_to_even_code_and_saturation():
    pos = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    got = oracle.e4m3_encode(mids)
    lo = np.arange(126)
    np.testing.assert_array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    # just off the midpoints: nearest wins
    np.testing.assert_array_equal(oracle.e4m3_encode(np.nextafter(mids, 0)), lo)
    np.testing.assert_array_equal(oracle.e4m3_encode(np.nextafter(mids, 1e9)), lo + 1)
    big = np.array([448.0, 449.0, 464.0, 480.0, 1e6, 1e300, np.inf])
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)


@pytest.mark.slow
def test_e4m3_quant_matches_torch_cast_exhaustively_below_448():
    """Every fp32 value in [2^-11, 448) (all 20 binades, 2^23 patterns each) plus 2^20
    patterns below, against PyTorch's CPU float8_e4m3fn cast (RNE); with inv_scale = 1
    the quantiser's fp32 multiply is exact, so this pins the codec."""
    lo_bits = np.float32(2.0 ** -11).view(np.uint32)
    hi_bits = np.float32(448.0).view(np.uint32)
    step = 1 << 23
    for start in range(int(lo_bits), int(hi_bits), step):
        bits = np.arange(start, min(start + step, int(hi_bits)), dtype=np.uint32)
        v = bits.view(np.float32)
        got = oracle.quant_f32(v, 1.0)
        ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (v[bad[:5]], got[bad[:5]], ref[bad[:5]])
    tiny = np.concatenate([np.arange(int(lo_bits) - (1 << 20), int(lo_bits), dtype=np.uint32),
                           np.arange(0, 1 << 16, dtype=np.uint32)]).view(np.float32)
    ref = torch.from_numpy(tiny).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.quant_f32(tiny, 1.0), ref)
    neg = -np.linspace(0.001, 447.0, 100001, dtype=np.float32)
    ref = torch.from_numpy(neg).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.quant_f32(neg, 1.0), ref)


def test_quant_f32_multiplies_in_fp32_before_rounding():
    """code = Q(fp32(u * inv)): u, inv are chosen so that the exact product lies just above
    the 1.0 / 1.125 midpoint (1.0625) while its fp32 rounding is the midpoint itself; the
    fp32 route ties to the even code 0x38, a binary64 product would give 0x39."""
    inv = np.float32(1.0) + np.float32(2.0 ** -23)
    u = np.float32(1.0625) / inv
    found = None
    for _ in range(64):
        exact = float(u) * float(inv)            # exact: 24-bit x 24-bit fits binary64
        if np.float32(exact) == np.float32(1.0625) and exact > 1.0625:
            found = u
            break
        u = np.nextafter(u, np.float32(2.0))
    assert found is not None
    assert oracle.e4m3_encode(np.array([float(found) * float(inv)]))[0] == 0x39
    assert oracle.quant_f32(np.array([found], dtype=np.float32), float(inv))[0] == 0x38


def test_fp8_products_exact_against_int64():
    """sum_k dec(a) dec(b) in binary64 equals the int64 sum in units of 2^-18 bit for bit:
    products are integers < 2^36 in those units and 4096-term sums stay < 2^48."""
    rng = np.random.default_rng(9)
    valid = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    a = rng.choice(valid, (16, 4096))
    b = rng.choice(valid, (24, 4096))
    a[0, :] = 0x7E
    b[0, :] = 0x7E                      # 4096 * 448^2: the largest possible sum
    got = oracle.matmul_nt(oracle.e4m3_decode(a), oracle.e4m3_decode(b))
    ia, ib = e4m3_int(a), e4m3_int(b)
    ref = ia @ ib.T                       # int64, exact
    np.testing.assert_array_equal(got * 2.0 ** 18, ref.astype(np.float64))
    assert np.all(np.abs(ref) < 2 ** 53)
    assert got[0, 0] == 4096 * 448.0 * 448.0


def test_fp8_pipeline_codes_are_post_relu_and_in_range():
    inp = workloads.generate(workloads.workload(4, m=37, n=29, k=64))
    codes, u = oracle.fp8_gemm_bn_relu_quant(inp)
    assert codes.shape == (37, 29) and np.all(u >= 0)
    assert np.all(codes <= 0x7E)
    np.testing.assert_array_equal(codes, oracle.e4m3_encode(u / inp["s_y"]))
    np.testing.assert_array_equal(codes[u == 0], 0)


def test_fp8_pipeline_with_gelu_forms():
    """Quantised MatMul + GELU ([RFC] §2.1): rebuilt from the exact integer e4m3 products, BN in
    numpy and each GELU form from an independent definition (scipy's normal CDF; the tanh
    formula); the codes are the codec applied to u / s_y, signed where u < 0."""
    from scipy.stats import norm
    inp = workloads.generate(workloads.workload(4, m=19, n=24, k=64))
    y = (e4m3_int(inp["x"]) @ e4m3_int(inp["w"]).T).astype(np.float64) * 2.0 ** -18 * inp["s_x"] * inp["s_w"]
    g, b, mu, var = (np.asarray(inp[k], np.float64) for k in ("gamma", "beta", "mean", "var"))
    z = g * (y - mu) / np.sqrt(var + inp["eps"]) + b
    forms = {"gelu_erf": lambda t: t * norm.cdf(t),
             "gelu_tanh": lambda t: 0.5 * t * (1 + np.tanh(np.sqrt(2 / np.pi) * (t + 0.044715 * t ** 3)))}
    for act, f in forms.items():
        codes, u = oracle.fp8_gemm_bn_act_quant(inp, act)
        np.testing.assert_allclose(u, f(z), rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(codes, oracle.e4m3_encode(u / inp["s_y"]))
        neg = u / inp["s_y"] < -2.0 ** -10          # below half the smallest subnormal: a signed code
        assert np.any(neg) and np.all(codes[neg] & 0x80)
    codes, u = oracle.fp8_gemm_bn_act_quant(inp, "relu")
    c2, u2 = oracle.fp8_gemm_bn_relu_quant(inp)
    np.testing.assert_array_equal(codes, c2)


def test_metric_floor():
    o = np.array([0.0, 1.0, -1.0, 0.0])
    assert oracle.rel_error(o, o) == 0.0
    # 1-D: one channel, floor = rms(o) = sqrt(0.5)
    assert math.isclose(oracle.rel_error(o + np.array([0.1, 0, 0, 0]), o), 0.1 / math.sqrt(0.5))
    # 2-D: the floor is the rms of each column (channel)
    o2 = np.array([[0.0, 10.0], [0.0, -10.0], [1.0, 0.0], [-1.0, 0.0]])
    g2 = o2 + np.array([[0.5, 0.0], [0, 0], [0, 0], [0, 0]])
    assert math.isclose(oracle.rel_error(g2, o2), 0.5 / math.sqrt(0.5))
    g3 = o2 + np.array([[0.0, 0.0], [0, 0], [0, 1.0], [0, 0]])
    assert math.isclose(oracle.rel_error(g3, o2), 1.0 / math.sqrt(50.0))


def test_round_bf16_single_rounding_ties_and_range():
    """bf16 storage rounding from binary64: agrees with torch's fp32 -> bf16 cast (round to
    nearest even) wherever the value is an fp32 value, and with exact rational arithmetic on
    arbitrary binary64 values; ties go to the even significand; one rounding, not two."""
    from fractions import Fraction
    rng = np.random.default_rng(21)
    f32 = np.concatenate([rng.standard_normal(5000), rng.standard_normal(500) * 1e30,
                          rng.standard_normal(500) * 1e-39, [0.0, -0.0, 1.0, -2.5]]).astype(np.float32)
    want = torch.from_numpy(f32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(f32.astype(np.float64)), want)
    # exact: the two bf16 neighbours of v from its binary expansion, the nearer (ties even)
    v = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000),
                        1.0 + rng.integers(0, 1 << 10, 200) * 2.0 ** -10])
    got = oracle.round_bf16(v)
    for x, gx in zip(v, got):
        fx = Fraction(float(x))
        e = abs(fx).numerator.bit_length() - abs(fx).denominator.bit_length()
        while Fraction(2) ** e > abs(fx):
            e -= 1
        while Fraction(2) ** (e + 1) <= abs(fx):
            e += 1
        ulp = Fraction(2) ** max(e - 7, -133)
        lo = (fx / ulp).__floor__()
        r = fx / ulp - lo
        k = lo + (1 if r > Fraction(1, 2) or (r == Fraction(1, 2) and lo % 2 == 1) else 0)
        assert Fraction(float(gx)) == k * ulp, x
    one = 1.0
    cases = {one + 2.0 ** -8: one,                            # tie -> even (1.0)
             one + 3 * 2.0 ** -8: one + 2.0 ** -6,            # tie -> even (mantissa 2)
             -(one + 2.0 ** -8): -one,
             one + 2.0 ** -8 + 2.0 ** -30: one + 2.0 ** -7,   # just above the tie: up
             2.0 ** 128 - 2.0 ** 119 - 2.0 ** 100: 2.0 ** 128 - 2.0 ** 120,   # largest finite
             2.0 ** 128 - 2.0 ** 119: np.inf,                 # tie at the top goes to 2^128
             2.0 ** -134: 0.0, 3 * 2.0 ** -134: 2.0 ** -132}  # subnormal ties
    for x, want in cases.items():
        assert oracle.round_bf16(np.array([x]))[0] == want, x
    # one rounding: via fp32, 1 + 2^-8 + 2^-30 would land on the tie and go down to 1.0
    assert float(np.float32(one + 2.0 ** -8 + 2.0 ** -30)) == one + 2.0 ** -8


def test_ffn_against_pure_python_loops():
    """FC1 -> activation -> FC2 (+ b2, + residual) on a tiny block, against plain Python loops
    over the definition (no numpy, no oracle kernels): h_f = act(sum_d x_d W1[f][d] + b1_f),
    y_j = sum_f h_f W2[j][f] + b2_j + r_j; with ReLU and with the tanh GELU."""
    for act in ("relu", "gelu_tanh"):
        wl = workloads.FfnWorkload("tiny", m=3, d_model=5, d_ff=7, act=act, residual=True, seed=9)
        inp = workloads.generate(wl)
        got = oracle.ffn(inp)
        x = oracle.widen(inp["x"], "bf16").tolist()
        w1 = oracle.widen(inp["w1"], "bf16").tolist()
        w2 = oracle.widen(inp["w2"], "bf16").tolist()
        r = oracle.widen(inp["residual"], "bf16").tolist()
        b1 = [float(v) for v in inp["b1"]]
        b2 = [float(v) for v in inp["b2"]]
        for t in range(3):
            h = []
            for f in range(7):
                u = sum(x[t][d] * w1[f][d] for d in range(5)) + b1[f]
                if act == "relu":
                    h.append(max(u, 0.0))
                else:
                    h.append(0.5 * u * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3))))
            for j in range(5):
                want = sum(h[f] * w2[j][f] for f in range(7)) + b2[j] + r[t][j]
                assert abs(got[t][j] - want) <= 1e-12 * (1.0 + abs(want))
        # rows select tokens
        np.testing.assert_array_equal(oracle.ffn(inp, rows=[2, 0]), got[[2, 0]])
