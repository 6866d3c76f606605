"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances (the floored relative metric of oracle.rel_error):
  fp32 1e-4, bf16 2e-2; fp8 outputs within one e4m3 code of the oracle's code;
  the quantiser bit-exact on identical fp32 inputs.
Every output buffer carries a guard band after its end that must stay untouched.
"""
import os

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

TOL = {"f32": 1e-4, "bf16": 2e-2}
# The unfused comparison chain stores up to three bf16 intermediates (conv output, BN
# output, residual sum) where the fused kernel keeps fp32 registers; each rounding is
# amplified by the channel's BN scale, so the chain gets twice the fused tolerance.
TOL_UNFUSED = {"f32": 1e-4, "bf16": 4e-2}
GUARD = 4096
CONV_TILES = (1, 2, 3)                 # the implicit GEMM's tiles: 128x128, 128x64, 64x64
GEMM_TILES = (0,) + CONV_TILES         # plus the dense GEMM's eight-wave 256x256


class _TuningEnv:
    """The DLF_* tuning switches: the library reads them once when it loads, so every change
    of the environment here is followed by dlf_tuning_reload()."""

    def __setitem__(self, key, val):
        os.environ[key] = val
        dlf().dlf_tuning_reload()

    def pop(self, key, default=None):
        r = os.environ.pop(key, default)
        dlf().dlf_tuning_reload()
        return r


ENV = _TuningEnv()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dl_fusion_amd  # noqa: F401  (loud failure if the library is missing)
    torch.cuda.set_device(0)
    yield
    ENV.pop("DLF_TILE", None)
    ENV.pop("DLF_CONV", None)


def dlf():
    import dl_fusion_amd
    return dl_fusion_amd


def layers():
    from dl_fusion_amd import layers as L
    return L


def case(msg):
    print(f"\n[case] {msg}", flush=True)


def guarded(shape, dtype):
    """A contiguous output tensor followed by a canary-filled guard band."""
    n = int(np.prod(shape))
    buf = torch.empty(n + GUARD, dtype=dtype, device="cuda")
    if dtype == torch.uint8:
        buf.fill_(0xA5)
    elif dtype == torch.bfloat16:
        buf.view(torch.int16).fill_(0x7FA5)
    else:
        buf.view(torch.int32).fill_(0x7FA5A5A5)
    return buf, buf[:n].view(shape)


def guard_intact(buf, n):
    tail = buf[n:]
    if buf.dtype == torch.uint8:
        return bool((tail == 0xA5).all())
    if buf.dtype == torch.bfloat16:
        return bool((tail.view(torch.int16) == 0x7FA5).all())
    return bool((tail.view(torch.int32) == 0x7FA5A5A5).all())


def host(t, dtype):
    return layers().to_host(t, dtype)


# ---------------------------------------------------------------------------
# Convolutions
# ---------------------------------------------------------------------------
def set_route(conv, tile):
    """conv: None = the library's own choice; "stream" = the halo kernel that streams weights
    per row tile, never the resident-weight or whole-image ones; "generic" = the implicit-GEMM
    kernel instead of any halo kernel; tile: force an MFMA tile of the implicit GEMM."""
    for key, val in (("DLF_CONV", conv), ("DLF_TILE", None if tile is None else str(tile))):
        if val is None:
            ENV.pop(key, None)
        else:
            ENV[key] = val


def check_conv(wl, tiles=(), unfused=True):
    """The default route, then (bf16) the generic implicit GEMM with its default tile and
    with every tile in `tiles`."""
    inp = workloads.generate(wl)
    ref = oracle.conv_bn_act(inp)
    L = layers().make_layer(inp, with_unfused=unfused)
    tdt = L.y.dtype
    routes = [(None, None)]
    if wl.dtype == "bf16":
        routes += [("stream", None), ("generic", None)] + [("generic", t) for t in tiles]
    try:
        for conv, tile in routes:
            set_route(conv, tile)
            case(f"conv_fused {wl} route={conv} tile={tile}")
            buf, y = guarded(L.out_shape, tdt)
            L.forward(y=y)
            torch.cuda.synchronize()
            got = oracle.widen(host(y, wl.dtype), wl.dtype)
            err = oracle.rel_error(got, ref)
            assert err <= TOL[wl.dtype], (wl, conv, tile, err)
            assert guard_intact(buf, y.numel()), "store beyond the output"
            if wl.act == "relu":
                assert np.all(got >= 0)
    finally:
        set_route(None, None)
    if unfused:
        case(f"conv_unfused {wl}")
        yu = L.forward_unfused()
        torch.cuda.synchronize()
        err = oracle.rel_error(oracle.widen(host(yu, wl.dtype), wl.dtype), ref)
        assert err <= TOL_UNFUSED[wl.dtype], ("unfused", wl, err)


def test_config0_fp32_conv_bn_relu_full():
    check_conv(workloads.workload(0))


def test_config1_bf16_conv_bn_relu_full():
    check_conv(workloads.workload(1))


def test_config2_bf16_conv_bn_residual_relu_full():
    check_conv(workloads.workload(2))


def test_config2_with_conv_bias_variant():
    check_conv(workloads.workload(2, n=4, conv_bias=True), unfused=False)


RAGGED_BF16 = [
    dict(n=2, h=9, w=7, cin=8, cout=40, kh=3, kw=3, stride=1, pad=1, act="relu", residual=False),
    dict(n=1, h=13, w=11, cin=24, cout=72, kh=3, kw=3, stride=2, pad=1, act="gelu_tanh", residual=True),
    dict(n=3, h=6, w=6, cin=64, cout=64, kh=1, kw=1, stride=1, pad=0, act="none", residual=False),
    dict(n=1, h=10, w=10, cin=16, cout=96, kh=5, kw=5, stride=1, pad=2, act="relu", residual=True),
    dict(n=2, h=7, w=9, cin=136, cout=33, kh=3, kw=3, stride=1, pad=1, act="relu", residual=False),
    dict(n=5, h=15, w=15, cin=32, cout=129, kh=3, kw=3, stride=1, pad=0, act="gelu_tanh", residual=False),
    dict(n=2, h=8, w=12, cin=48, cout=80, kh=3, kw=3, stride=2, pad=1, act="gelu_erf", residual=True),
]


@pytest.mark.parametrize("i", range(len(RAGGED_BF16)))
def test_bf16_conv_ragged_shapes_every_tile(i):
    wl = workloads.workload(1, conv_bias=bool(i % 2), **RAGGED_BF16[i])
    check_conv(wl, tiles=CONV_TILES, unfused=(i < 3))



# Unpadded strided 1x1 convolutions (a ResNet downsample) stream with their rows gathered:
# strides 2 and 3, odd and even image sides, one to three column blocks, K of 128 and 256,
# with and without activation and conv bias; forced onto the streaming kernel (DLF_GEMM=
# stream; its 128-wide column blocks, and 256-wide ones where they divide c_out), onto the
# implicit GEMM (DLF_GEMM=tiled, DLF_CONV=generic), and on the library's own choice (the last
# case is large enough for it to stream), each against the oracle.
STRIDED_1X1 = [
    dict(n=3, h=15, w=13, cin=256, cout=512, kh=1, kw=1, stride=2, pad=0, act="none", residual=False),
    dict(n=2, h=12, w=12, cin=128, cout=384, kh=1, kw=1, stride=2, pad=0, act="relu", residual=False),
    dict(n=1, h=17, w=20, cin=256, cout=256, kh=1, kw=1, stride=3, pad=0, act="gelu_erf", residual=False),
    dict(n=12, h=56, w=56, cin=256, cout=512, kh=1, kw=1, stride=2, pad=0, act="none", residual=False),
]


@pytest.mark.parametrize("i", range(len(STRIDED_1X1)))
def test_bf16_strided_1x1_streaming_route(i):
    wl = workloads.workload(1, conv_bias=bool(i % 2), **STRIDED_1X1[i])
    inp = workloads.generate(wl)
    ref = oracle.conv_bn_act(inp)
    L = layers().make_layer(inp, with_unfused=False)
    routes = [("stream", None, None), ("tiled", None, None), (None, "generic", None), (None, None, None)]
    if wl.cout % 256 == 0:
        routes.append(("stream", None, "256"))
    try:
        for gemm, conv, nb in routes:
            for key, val in (("DLF_GEMM", gemm), ("DLF_CONV", conv), ("DLF_STREAM_NB", nb)):
                if val is None:
                    ENV.pop(key, None)
                else:
                    ENV[key] = val
            case(f"conv_fused {wl} gemm={gemm} conv={conv} block={nb}")
            buf, y = guarded(L.out_shape, torch.bfloat16)
            L.forward(y=y)
            torch.cuda.synchronize()
            assert guard_intact(buf, y.numel()), "store beyond the output"
            err = oracle.rel_error(oracle.widen(host(y, "bf16"), "bf16"), ref)
            assert err <= TOL["bf16"], (wl, gemm, conv, nb, err)
    finally:
        for key in ("DLF_GEMM", "DLF_CONV", "DLF_STREAM_NB"):
            ENV.pop(key, None)

# Any number of input channels (Cin % 8 != 0): the implicit GEMM gathers both operands value
# by value.  The stem geometry (7x7, stride 2, pad 3, three channels), a ragged K of 27, one
# channel, and 5 or 12 channels with a residual and a stride.
ANYC_BF16 = [
    dict(n=2, h=23, w=21, cin=3, cout=64, kh=7, kw=7, stride=2, pad=3, act="relu", residual=False),
    dict(n=3, h=9, w=10, cin=5, cout=40, kh=3, kw=3, stride=1, pad=1, act="gelu_erf", residual=True),
    dict(n=4, h=6, w=7, cin=1, cout=33, kh=1, kw=1, stride=1, pad=0, act="none", residual=False),
    dict(n=1, h=13, w=11, cin=12, cout=72, kh=3, kw=3, stride=2, pad=1, act="relu", residual=True),
    dict(n=2, h=8, w=8, cin=3, cout=129, kh=3, kw=3, stride=1, pad=0, act="gelu_tanh", residual=False),
]


@pytest.mark.parametrize("i", range(len(ANYC_BF16)))
def test_bf16_conv_any_cin_every_tile(i):
    wl = workloads.workload(1, conv_bias=bool(i % 2), **ANYC_BF16[i])
    check_conv(wl, tiles=CONV_TILES, unfused=(i < 2))


# Up to four input channels with whole 16-byte input rows: the small-channel kernel (weights
# and the input patch re-laid in LDS with 4-channel pixels) by default, the value-by-value
# implicit GEMM on the forced generic route.  Ragged row tiles, a half channel block
# (Cout % 64 = 32), residuals, one and two channels, a tall image with many row tiles, and
# workgroups that run several rounds of compute and store waves.
SMALLC_BF16 = [
    dict(n=2, h=24, w=16, cin=3, cout=64, kh=7, kw=7, stride=2, pad=3, act="relu", residual=False),
    dict(n=3, h=10, w=8, cin=4, cout=96, kh=3, kw=3, stride=1, pad=1, act="gelu_erf", residual=True),
    dict(n=1, h=9, w=16, cin=2, cout=32, kh=5, kw=5, stride=2, pad=2, act="none", residual=True),
    dict(n=2, h=40, w=40, cin=1, cout=64, kh=3, kw=3, stride=1, pad=0, act="gelu_tanh", residual=False),
    dict(n=1, h=200, w=64, cin=3, cout=128, kh=7, kw=7, stride=2, pad=3, act="relu", residual=False),
    # several rounds of 16 fragments per workgroup (the shapes above plan one output row per
    # workgroup): two rounds with a residual at stride 1 (odd left padding, 8-byte patch
    # reads); two rounds with a 32-channel block at stride 2; five rounds with a shorter last
    # row tile; a 32-channel layer of two rounds
    dict(n=64, h=64, w=64, cin=3, cout=64, kh=3, kw=3, stride=1, pad=1, act="relu", residual=True),
    dict(n=64, h=64, w=72, cin=4, cout=96, kh=5, kw=5, stride=2, pad=2, act="gelu_tanh", residual=False),
    dict(n=64, h=96, w=96, cin=1, cout=64, kh=3, kw=3, stride=1, pad=0, act="gelu_erf", residual=True),
    dict(n=64, h=64, w=64, cin=2, cout=32, kh=3, kw=3, stride=1, pad=1, act="none", residual=False),
]


@pytest.mark.parametrize("i", range(len(SMALLC_BF16)))
def test_bf16_conv_small_channel_kernel(i):
    wl = workloads.workload(1, conv_bias=bool(i % 2), **SMALLC_BF16[i])
    check_conv(wl, tiles=(2,), unfused=(i < 2))


def test_resnet_stem_full_size_sampled():
    """The ResNet stem at batch 32: 224x224x3 -> 112x112x64, 7x7 stride 2 pad 3, BN, ReLU; 512
    sampled output pixels (the four corners among them) against the oracle."""
    wl = workloads.workload(1, n=32, h=224, w=224, cin=3, cout=64, kh=7, kw=7, stride=2, pad=3,
                            act="relu", residual=False)
    inp = workloads.generate(wl)
    L = layers().make_layer(inp, with_unfused=False)
    case(f"stem conv_fused {wl}")
    buf, y = guarded(L.out_shape, torch.bfloat16)
    L.forward(y=y)
    torch.cuda.synchronize()
    assert guard_intact(buf, y.numel())
    rng = np.random.default_rng(5)
    pts = np.stack([rng.integers(0, 32, 512), rng.integers(0, 112, 512), rng.integers(0, 112, 512)], 1)
    pts[:4] = [[0, 0, 0], [31, 111, 111], [0, 0, 111], [31, 111, 0]]
    ref = oracle.conv_bn_act(inp, pts=pts)
    got = oracle.widen(host(y, "bf16"), "bf16")[pts[:, 0], pts[:, 1], pts[:, 2], :]
    err = oracle.rel_error(got, ref)
    assert err <= TOL["bf16"], err
    assert np.all(got >= 0)


# 3x3 stride-1 pad-1 layers the halo kernel takes: several rows per workgroup with a
# shorter last row tile, one row per workgroup, 64 / 128 / 256 / 384 input channels,
# one or two 32-pixel fragments per wave, 48 KB and 96 KB halos.
HALO_BF16 = [
    dict(n=16, h=15, w=16, cin=64, cout=128, act="relu", residual=True),      # 2 rows, last 1
    dict(n=128, h=11, w=50, cin=64, cout=64, act="gelu_tanh", residual=False),  # 4 rows x 50, last 3
    dict(n=4, h=9, w=9, cin=128, cout=192, act="relu", residual=True),        # 1 row
    dict(n=2, h=5, w=6, cin=384, cout=64, act="none", residual=False),        # 1 row, 3 channel groups
    dict(n=64, h=14, w=14, cin=256, cout=64, act="relu", residual=True),      # 4 rows, last 2
    # 64 input channels with resident weights: one tile per workgroup with a residual, and
    # two output-channel tiles with up to three row tiles per workgroup
    dict(n=96, h=9, w=20, cin=64, cout=64, act="relu", residual=True),
    dict(n=320, h=2, w=8, cin=64, cout=128, act="gelu_tanh", residual=False),
    # small images, one image x 32 output channels per workgroup: 8 and 3 input channel groups
    dict(n=16, h=7, w=7, cin=512, cout=256, act="relu", residual=True),
    dict(n=48, h=13, w=11, cin=192, cout=96, act="gelu_tanh", residual=True),
    # 1x1 and 2x3 images: every tap but the centre (or nearly) reads padding.  One image is
    # not enough here: the metric floors each channel at its rms, and with one pixel per
    # channel the bf16-rounded folded weights alone reach 3% of a cancelled output.
    dict(n=64, h=1, w=1, cin=64, cout=64, act="relu", residual=False),
    dict(n=16, h=2, w=3, cin=64, cout=64, act="none", residual=True),
    # exact (erf) GELU through the resident-weight and the whole-image kernels (and, via the
    # forced routes, the streaming halo kernel and the implicit GEMM)
    dict(n=32, h=10, w=20, cin=64, cout=64, act="gelu_erf", residual=True),
    dict(n=64, h=7, w=7, cin=128, cout=64, act="gelu_erf", residual=False),
    # small images with 64 to 320 input channels, one to five 64-channel groups, ragged row
    # tiles, three output-channel tiles, a one-row image 128 wide, and 121-pixel images
    dict(n=3, h=9, w=13, cin=192, cout=128, act="relu", residual=True),
    dict(n=2, h=16, w=16, cin=128, cout=64, act="none", residual=False),
    dict(n=2, h=12, w=11, cin=320, cout=192, act="gelu_tanh", residual=True),
    dict(n=5, h=8, w=9, cin=64, cout=128, act="relu", residual=False),
    dict(n=2, h=1, w=128, cin=64, cout=64, act="relu", residual=True),
    dict(n=64, h=11, w=11, cin=128, cout=128, act="gelu_erf", residual=False),
]


@pytest.mark.parametrize("i", range(len(HALO_BF16)))
def test_bf16_conv_halo_shapes(i):
    wl = workloads.workload(1, conv_bias=bool(i % 2), kh=3, kw=3, stride=1, pad=1, **HALO_BF16[i])
    check_conv(wl, unfused=(i == 0))


RAGGED_F32 = [
    dict(n=2, h=9, w=7, cin=3, cout=5, kh=3, kw=3, stride=2, pad=1, act="relu", residual=False),
    dict(n=1, h=5, w=5, cin=16, cout=70, kh=1, kw=1, stride=1, pad=0, act="gelu_tanh", residual=True),
    dict(n=3, h=11, w=6, cin=7, cout=33, kh=5, kw=3, stride=1, pad=2, act="none", residual=False),
    dict(n=2, h=6, w=9, cin=12, cout=40, kh=3, kw=3, stride=1, pad=1, act="gelu_erf", residual=True),
    # the register-weight path at its largest K (252) with stride 2, and a 1x1 with K = 4
    dict(n=3, h=13, w=10, cin=28, cout=96, kh=3, kw=3, stride=2, pad=1, act="gelu_tanh", residual=False),
    dict(n=2, h=7, w=5, cin=4, cout=31, kh=1, kw=1, stride=1, pad=0, act="relu", residual=True),
    # K = 260 just past it (the sliced kernel)
    dict(n=1, h=6, w=6, cin=52, cout=20, kh=1, kw=5, stride=1, pad=2, act="relu", residual=False),
    # the register-weight path's 8- and 16-pixel workgroups, the second with a one-pixel tail
    dict(n=2, h=16, w=16, cin=8, cout=24, kh=3, kw=3, stride=1, pad=1, act="relu", residual=True),
    dict(n=1, h=33, w=33, cin=4, cout=16, kh=3, kw=3, stride=1, pad=1, act="gelu_tanh", residual=False),
]


@pytest.mark.parametrize("i", range(len(RAGGED_F32)))
def test_f32_conv_ragged_shapes(i):
    wl = workloads.workload(0, conv_bias=bool(i % 2), **RAGGED_F32[i])
    check_conv(wl)


def test_conv_empty_and_degenerate():
    d = dlf()
    case("conv empty batch")
    x = torch.empty(0, device="cuda", dtype=torch.bfloat16)
    d.dlf_conv_fused(d.conv_desc(0, 8, 8, 16, 16), x, x, None, None, x)
    case("conv eps=1e-2 no-bias stress at tiny size")
    check_conv(workloads.workload(2, n=1, h=3, w=3, cin=8, cout=32))


# ---------------------------------------------------------------------------
# bf16 GEMM + bias + activation
# ---------------------------------------------------------------------------
def gemm_reference(inp, rows, residual=None):
    wl = inp["workload"]
    x = oracle.widen(inp["x"], "bf16")[rows]
    y = oracle.matmul_nt(x, oracle.widen(inp["w"], "bf16"))
    if inp.get("bias") is not None:
        y = oracle.bias_add(y, inp["bias"])
    if residual is not None:
        y = oracle.add(y, oracle.widen(residual, "bf16")[rows])
    return oracle.activation(y, wl.act)


def sample_rows(m, tile=256, extra=40, seed=0):
    """Rows 0, 1, m-2, m-1, both rows at every tile edge, and `extra` random rows."""
    rng = np.random.default_rng(seed)
    edges = {0, 1, m - 1, m - 2}
    for t in range(tile, m, tile):
        edges.update({t - 1, t})
    edges = {r for r in edges if 0 <= r < m}
    return np.array(sorted(edges | set(rng.choice(m, min(extra, m), replace=False).tolist())))


def test_config3_bf16_gemm_bias_gelu_full_size_sampled():
    wl = workloads.workload(3)
    inp = workloads.generate(wl)
    L = layers().make_layer(inp)
    case(f"gemm_fused {wl}")
    buf, y = guarded((wl.m, wl.n), torch.bfloat16)
    L.forward(y=y)
    torch.cuda.synchronize()
    assert guard_intact(buf, y.numel())
    rows = sample_rows(wl.m)
    got_all = oracle.widen(host(y, "bf16"), "bf16")
    assert np.all(np.isfinite(got_all)) and got_all.min() >= -0.1701   # GELU(tanh) minimum ~ -0.170
    ref = gemm_reference(inp, rows)
    err = oracle.rel_error(got_all[rows], ref)
    assert err <= TOL["bf16"], err
    case("gemm_unfused config 3")
    yu = L.forward_unfused()
    torch.cuda.synchronize()
    err_u = oracle.rel_error(oracle.widen(host(yu, "bf16"), "bf16")[rows], ref)
    assert err_u <= TOL_UNFUSED["bf16"], err_u


RAGGED_GEMM = [
    dict(m=300, n=200, k=136, act="gelu_tanh", bias=True),
    dict(m=1, n=17, k=8, act="relu", bias=True),
    dict(m=513, n=257, k=520, act="none", bias=False),
    dict(m=64, n=48, k=0, act="gelu_tanh", bias=True),
    dict(m=777, n=1000, k=1024, act="relu", bias=True),
    dict(m=130, n=72, k=64, act="gelu_erf", bias=True),
]


@pytest.mark.parametrize("i", range(len(RAGGED_GEMM)))
def test_bf16_gemm_ragged_shapes_every_tile(i):
    wl = workloads.workload(3, **RAGGED_GEMM[i])
    inp = workloads.generate(wl)
    res = None
    if i % 2 == 0:
        res = workloads.bf16_bits(np.random.default_rng(i).standard_normal((wl.m, wl.n)).astype(np.float32))
    rows = np.arange(wl.m)
    ref = gemm_reference(inp, rows, res)
    L = layers().make_layer(inp)
    res_d = layers().to_device(res, "bf16") if res is not None else None
    for tile in (None,) + GEMM_TILES:
        if tile is None:
            ENV.pop("DLF_TILE", None)
        else:
            ENV["DLF_TILE"] = str(tile)
        case(f"gemm_fused {wl} tile={tile} residual={res is not None}")
        buf, y = guarded((wl.m, wl.n), torch.bfloat16)
        L.forward(y=y, residual=res_d)
        torch.cuda.synchronize()
        assert guard_intact(buf, y.numel())
        err = oracle.rel_error(oracle.widen(host(y, "bf16"), "bf16"), ref)
        assert err <= TOL["bf16"], (wl, tile, err)
    ENV.pop("DLF_TILE", None)
    if res is None:
        case(f"gemm_unfused {wl}")
        yu = L.forward_unfused()
        torch.cuda.synchronize()
        assert oracle.rel_error(oracle.widen(host(yu, "bf16"), "bf16"), ref) <= TOL_UNFUSED["bf16"]


# Memory-bound shapes take the streaming kernel (B in registers, A and the residual through
# an LDS ring of whole tiles): every (N, K) it is built for, at one and two workgroups a CU,
# ragged row counts (one row, a partial last tile, fewer tiles than workgroups, many tiles
# per workgroup), every activation, with and without residual and bias; forced onto it
# (DLF_GEMM=stream), onto the tiled kernel, and on the library's own choice, each against the
# oracle.
STREAM_GEMM = [
    dict(m=100, n=128, k=256, act="relu", bias=True),
    dict(m=1, n=128, k=128, act="gelu_tanh", bias=True),
    dict(m=9000, n=128, k=256, act="none", bias=False),
    dict(m=777, n=256, k=128, act="gelu_erf", bias=True),
    dict(m=33, n=256, k=256, act="relu", bias=True),
    dict(m=12345, n=384, k=128, act="gelu_tanh", bias=True),
    dict(m=4100, n=384, k=128, act="relu", bias=True),
    dict(m=40000, n=128, k=256, act="relu", bias=True),        # the library's own choice takes
    dict(m=20000, n=256, k=128, act="gelu_tanh", bias=True),   # these two (4M outputs or more)
    # N K = 32768 from 2048 tiles: two workgroups a CU (half the ring each)
    dict(m=70001, n=128, k=256, act="gelu_erf", bias=True),
    dict(m=66000, n=256, k=128, act="relu", bias=False),
    # wider outputs in column blocks, several workgroups a row tile: 2 x 256, 5 x 128 (a
    # block count that is no power of two), 3 x 256 at K = 256, and 2 x 256 at two a CU
    dict(m=5000, n=512, k=128, act="relu", bias=True),
    dict(m=3001, n=640, k=128, act="gelu_tanh", bias=True),
    dict(m=2500, n=768, k=256, act="none", bias=True),
    dict(m=70001, n=512, k=128, act="gelu_erf", bias=False),
]


@pytest.mark.parametrize("res", [False, True])
@pytest.mark.parametrize("i", range(len(STREAM_GEMM)))
def test_bf16_gemm_streaming_route(i, res):
    wl = workloads.workload(3, **STREAM_GEMM[i])
    inp = workloads.generate(wl)
    r = None
    if res:
        r = workloads.bf16_bits(np.random.default_rng(90 + i).standard_normal((wl.m, wl.n)).astype(np.float32))
    ref = gemm_reference(inp, np.arange(wl.m), r)
    L = layers().make_layer(inp, with_unfused=False)
    r_d = layers().to_device(r, "bf16") if r is not None else None
    try:
        for route in ("stream", "tiled", None):
            if route is None:
                ENV.pop("DLF_GEMM", None)
            else:
                ENV["DLF_GEMM"] = route
            case(f"gemm_fused {wl} route={route} residual={res}")
            buf, y = guarded((wl.m, wl.n), torch.bfloat16)
            L.forward(y=y, residual=r_d)
            torch.cuda.synchronize()
            assert guard_intact(buf, y.numel())
            err = oracle.rel_error(oracle.widen(host(y, "bf16"), "bf16"), ref)
            assert err <= TOL["bf16"], (wl, route, err)
    finally:
        ENV.pop("DLF_GEMM", None)



@pytest.mark.parametrize("nb,n,k", [(128, 512, 128), (128, 768, 256), (256, 768, 128)])
def test_bf16_gemm_streaming_forced_block_width(nb, n, k):
    """Column blocks narrower than the widest that divides N (DLF_STREAM_NB), with residual."""
    wl = workloads.workload(3, m=4097, n=n, k=k, act="relu", bias=True)
    inp = workloads.generate(wl)
    r = workloads.bf16_bits(np.random.default_rng(7).standard_normal((wl.m, wl.n)).astype(np.float32))
    ref = gemm_reference(inp, np.arange(wl.m), r)
    L = layers().make_layer(inp, with_unfused=False)
    r_d = layers().to_device(r, "bf16")
    ENV["DLF_GEMM"] = "stream"
    ENV["DLF_STREAM_NB"] = str(nb)
    try:
        case(f"gemm_fused {wl} route=stream block={nb} residual=True")
        buf, y = guarded((wl.m, wl.n), torch.bfloat16)
        L.forward(y=y, residual=r_d)
        torch.cuda.synchronize()
        assert guard_intact(buf, y.numel())
        err = oracle.rel_error(oracle.widen(host(y, "bf16"), "bf16"), ref)
        assert err <= TOL["bf16"], (wl, nb, err)
    finally:
        ENV.pop("DLF_GEMM", None)
        ENV.pop("DLF_STREAM_NB", None)

# Rows of 8 MB or more are past the 32-bit offsets of the buffer-resource loads: the library
# reads them with 64-bit global addresses and the basic tiles (a tuned tile falls back to
# 256 x 256).  One K just past that limit per input type, on the default, a tuned and a small
# tile; the fp8 case draws small e4m3 codes directly, with an output scale that keeps the
# codes unsaturated.
WIDE_K = [
    (3, dict(m=3, n=40, k=(1 << 22) + 32, act="gelu_tanh", bias=True)),
    (4, dict(m=3, n=40, k=(1 << 23) + 16, out_scale=128.0)),
]


def wide_fp8_inputs(wl):
    """fp8 inputs at a very large K without quantising normals (slow at this size): e4m3 codes
    of magnitude 0.5 .. 1.875 with random signs, unit scales, and the BN parameters the seeded
    generator draws for the same output channels."""
    inp = workloads.generate(workloads.workload(4, m=wl.m, n=wl.n, k=16))
    rng = np.random.Generator(np.random.PCG64(wl.seed + 1))
    def codes(shape):
        return (rng.integers(0x30, 0x40, shape, dtype=np.uint8) | (rng.integers(0, 2, shape, dtype=np.uint8) << 7))
    inp.update(workload=wl, x=codes((wl.m, wl.k)), w=codes((wl.n, wl.k)), s_x=1.0, s_w=1.0,
               s_y=float(np.float32(wl.out_scale)))
    return inp


@pytest.mark.parametrize("i", range(len(WIDE_K)))
def test_gemm_rows_past_the_buffer_range(i):
    idx, over = WIDE_K[i]
    wl = workloads.workload(idx, **over)
    inp = workloads.generate(wl) if idx == 3 else wide_fp8_inputs(wl)
    rows = np.arange(wl.m)
    ref = gemm_reference(inp, rows) if idx == 3 else fp8_reference(inp, rows)[0]
    L = layers().make_layer(inp, with_unfused=False)
    for tile in (None, 0, 1):
        if tile is None:
            ENV.pop("DLF_TILE", None)
        else:
            ENV["DLF_TILE"] = str(tile)
        case(f"wide-row gemm {wl} tile={tile}")
        dt = torch.bfloat16 if idx == 3 else torch.uint8
        buf, y = guarded((wl.m, wl.n), dt)
        L.forward(y=y)
        torch.cuda.synchronize()
        assert guard_intact(buf, y.numel())
        if idx == 3:
            err = oracle.rel_error(oracle.widen(host(y, "bf16"), "bf16"), ref)
            assert err <= TOL["bf16"], (tile, err)
        else:
            assert_codes_within_one(host(y, "fp8"), ref)
    ENV.pop("DLF_TILE", None)


# ---------------------------------------------------------------------------
# One GEMM over concatenated weights, stored split by columns ([OPPL] §3.2, Q/K/V)
# ---------------------------------------------------------------------------
SPLIT_GEMM = [
    (3, dict(m=300, n=3 * 136, k=136, act="none", bias=True)),       # Q, K, V; ragged rows
    (2, dict(m=77, n=2 * 64, k=520, act="gelu_erf", bias=False)),
    (4, dict(m=513, n=4 * 256, k=64, act="relu", bias=True)),        # parts meet at tile borders
    (3, dict(m=64, n=3 * 88, k=0, act="none", bias=True)),           # k = 0: bias only
]


@pytest.mark.parametrize("i", range(len(SPLIT_GEMM)))
def test_bf16_gemm_split_store_every_tile(i):
    parts, over = SPLIT_GEMM[i]
    wl = workloads.workload(3, **over)
    inp = workloads.generate(wl)
    refs = oracle.gemm_bias_act_split(inp, parts)
    L = layers().make_layer(inp, with_unfused=False)
    pc = wl.n // parts
    for tile in (None,) + GEMM_TILES:
        if tile is None:
            ENV.pop("DLF_TILE", None)
        else:
            ENV["DLF_TILE"] = str(tile)
        case(f"gemm_fused_split {wl} parts={parts} tile={tile}")
        outs = [guarded((wl.m, pc), torch.bfloat16) for _ in range(parts)]
        dlf().dlf_gemm_fused_split(L.desc, L.x, L.w, None, L.bias, [y for _, y in outs])
        torch.cuda.synchronize()
        for p, ((buf, y), ref) in enumerate(zip(outs, refs)):
            assert guard_intact(buf, y.numel()), p
            err = oracle.rel_error(oracle.widen(host(y, "bf16"), "bf16"), ref)
            assert err <= TOL["bf16"], (tile, p, err)
    ENV.pop("DLF_TILE", None)


# ---------------------------------------------------------------------------
# Gated projections: SwiGLU and GELU x Mul over interleaved (gate, up) rows ([RFC] §2.2 - §2.4)
# ---------------------------------------------------------------------------
GATED_GEMM = [
    ("silu", dict(m=300, n=2 * 136, k=136, act="none", bias=True)),
    ("gelu_tanh", dict(m=77, n=2 * 100, k=520, act="none", bias=False)),   # 100 outputs: chunk tail
    ("gelu_erf", dict(m=513, n=2 * 256, k=64, act="none", bias=True)),
    ("silu", dict(m=64, n=2 * 24, k=0, act="none", bias=True)),
]


@pytest.mark.parametrize("i", range(len(GATED_GEMM)))
def test_bf16_gemm_gated_every_tile(i):
    gate, over = GATED_GEMM[i]
    wl = workloads.workload(3, **over)
    inp = workloads.generate(wl)
    ref = oracle.gemm_gated(inp, gate)
    L = layers().make_layer(inp, with_unfused=False)
    d = dlf()
    desc = d.gemm_desc(wl.m, wl.n, wl.k, "bf16", "bf16", "none")
    for tile in (None,) + GEMM_TILES:
        if tile is None:
            ENV.pop("DLF_TILE", None)
        else:
            ENV["DLF_TILE"] = str(tile)
        case(f"gemm_fused_gated {gate} {wl} tile={tile}")
        buf, y = guarded((wl.m, wl.n // 2), torch.bfloat16)
        d.dlf_gemm_fused_gated(desc, L.x, L.w, None, L.bias, gate, y)
        torch.cuda.synchronize()
        assert guard_intact(buf, y.numel())
        err = oracle.rel_error(oracle.widen(host(y, "bf16"), "bf16"), ref)
        assert err <= TOL["bf16"], (tile, err)
    ENV.pop("DLF_TILE", None)


def test_qkv_projection_full_size_sampled():
    """The LLaMA-7B Q/K/V projections as one 4096 x 12288 x 4096 GEMM stored as Q, K and V."""
    wl = workloads.workload(3, n=3 * 4096, act="none", bias=True)
    inp = workloads.generate(wl)
    L = layers().make_layer(inp, with_unfused=False)
    case(f"qkv {wl}")
    outs = [guarded((wl.m, 4096), torch.bfloat16) for _ in range(3)]
    dlf().dlf_gemm_fused_split(L.desc, L.x, L.w, None, L.bias, [y for _, y in outs])
    torch.cuda.synchronize()
    rows = sample_rows(wl.m)
    refs = oracle.gemm_bias_act_split(inp, 3, rows)
    for p, ((buf, y), ref) in enumerate(zip(outs, refs)):
        assert guard_intact(buf, y.numel()), p
        err = oracle.rel_error(oracle.widen(host(y, "bf16"), "bf16")[rows], ref)
        assert err <= TOL["bf16"], (p, err)


def test_fp8_gemm_split_store():
    wl = workloads.workload(4, m=77, n=2 * 64, k=144)
    inp = workloads.generate(wl)
    codes, _ = fp8_reference(inp, np.arange(wl.m))
    L = layers().make_layer(inp, with_unfused=False)
    for tile in (None, 0, 3):
        if tile is None:
            ENV.pop("DLF_TILE", None)
        else:
            ENV["DLF_TILE"] = str(tile)
        case(f"fp8 split {wl} tile={tile}")
        outs = [guarded((wl.m, 64), torch.uint8) for _ in range(2)]
        dlf().dlf_gemm_fused_split(L.desc, L.x, L.w, L.alpha, L.shift, [y for _, y in outs])
        torch.cuda.synchronize()
        for p, (buf, y) in enumerate(outs):
            assert guard_intact(buf, y.numel()), p
            assert_codes_within_one(host(y, "fp8"), codes[:, 64 * p:64 * (p + 1)])
    ENV.pop("DLF_TILE", None)


# ---------------------------------------------------------------------------
# fp8 GEMM + scale/shift + ReLU + static e4m3 quantisation
# ---------------------------------------------------------------------------
def fp8_reference(inp, rows):
    sub = dict(inp)
    codes, u = oracle.fp8_gemm_bn_relu_quant(sub, rows=rows)
    return codes, u


def assert_codes_within_one(got, ref):
    d = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    assert np.all(got <= 0x7E) and np.all(ref <= 0x7E)
    assert d.max() <= 1, (d.max(), np.argwhere(d > 1)[:5])
    return float(np.mean(d == 0))


def test_config4_fp8_gemm_bn_relu_quant_full_size_sampled():
    wl = workloads.workload(4)
    inp = workloads.generate(wl)
    L = layers().make_layer(inp)
    case(f"fp8_fused {wl}")
    buf, y = guarded((wl.m, wl.n), torch.uint8)
    L.forward(y=y)
    torch.cuda.synchronize()
    assert guard_intact(buf, y.numel())
    got_all = host(y, "fp8")
    assert np.all(got_all <= 0x7E)          # non-negative finite codes only (post-ReLU, saturating)
    rows = sample_rows(wl.m)
    ref, _ = fp8_reference(inp, rows)
    exact = assert_codes_within_one(got_all[rows], ref)
    assert exact > 0.9, exact
    case("fp8_unfused config 4")
    yu = L.forward_unfused()
    torch.cuda.synchronize()
    assert_codes_within_one(host(yu, "fp8")[rows], ref)


RAGGED_FP8 = [
    dict(m=300, n=200, k=144),
    dict(m=77, n=33, k=16),
    dict(m=513, n=260, k=1040),
    dict(m=1000, n=1100, k=4096),
]


@pytest.mark.parametrize("i", range(len(RAGGED_FP8)))
def test_fp8_gemm_ragged_shapes_every_tile(i):
    wl = workloads.workload(4, **RAGGED_FP8[i])
    inp = workloads.generate(wl)
    rows = np.arange(wl.m)
    ref, u = fp8_reference(inp, rows)
    L = layers().make_layer(inp)
    for tile in (None,) + GEMM_TILES:
        if tile is None:
            ENV.pop("DLF_TILE", None)
        else:
            ENV["DLF_TILE"] = str(tile)
        case(f"fp8_fused {wl} tile={tile}")
        buf, y = guarded((wl.m, wl.n), torch.uint8)
        L.forward(y=y)
        torch.cuda.synchronize()
        assert guard_intact(buf, y.numel())
        assert_codes_within_one(host(y, "fp8"), ref)
    ENV.pop("DLF_TILE", None)
    case(f"fp8 -> bf16 out {wl}")
    d = dlf()
    yb = torch.empty((wl.m, wl.n), dtype=torch.bfloat16, device="cuda")
    d.dlf_gemm_fused(d.gemm_desc(wl.m, wl.n, wl.k, "fp8", "bf16", "relu"), L.x, L.w, L.alpha, L.shift, None, yb)
    torch.cuda.synchronize()
    assert oracle.rel_error(oracle.widen(host(yb, "bf16"), "bf16"), u) <= TOL["bf16"]
    case(f"fp8_unfused {wl}")
    yu = L.forward_unfused()
    torch.cuda.synchronize()
    assert_codes_within_one(host(yu, "fp8"), ref)


def signed_code_order(codes):
    """e4m3 codes in value order: sign-magnitude to a signed integer, with -0 equal to +0."""
    c = codes.astype(np.int32)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


@pytest.mark.parametrize("act", ["gelu_tanh", "gelu_erf"])
def test_fp8_gemm_gelu_every_tile(act):
    """Quantised MatMul + GELU ([RFC] §2.1): e4m3 codes (signed: GELU dips below zero) within one
    code of the oracle's, and the bf16 form within the bf16 tolerance."""
    wl = workloads.workload(4, m=300, n=200, k=144)
    inp = workloads.generate(wl)
    codes, u = oracle.fp8_gemm_bn_act_quant(inp, act)
    assert np.any(codes & 0x80)
    L = layers().make_layer(inp, with_unfused=False)
    d = dlf()
    desc8 = d.gemm_desc(wl.m, wl.n, wl.k, "fp8", "fp8", act, L.inv_s_y)
    desc16 = d.gemm_desc(wl.m, wl.n, wl.k, "fp8", "bf16", act)
    for tile in (None,) + GEMM_TILES:
        if tile is None:
            ENV.pop("DLF_TILE", None)
        else:
            ENV["DLF_TILE"] = str(tile)
        case(f"fp8 {act} {wl} tile={tile}")
        buf, y = guarded((wl.m, wl.n), torch.uint8)
        d.dlf_gemm_fused(desc8, L.x, L.w, L.alpha, L.shift, None, y)
        torch.cuda.synchronize()
        assert guard_intact(buf, y.numel())
        diff = np.abs(signed_code_order(host(y, "fp8")) - signed_code_order(codes))
        assert diff.max() <= 1, (tile, diff.max())
    ENV.pop("DLF_TILE", None)
    case(f"fp8 {act} -> bf16 {wl}")
    yb = torch.empty((wl.m, wl.n), dtype=torch.bfloat16, device="cuda")
    d.dlf_gemm_fused(desc16, L.x, L.w, L.alpha, L.shift, None, yb)
    torch.cuda.synchronize()
    assert oracle.rel_error(oracle.widen(host(yb, "bf16"), "bf16"), u) <= TOL["bf16"]


def test_fp8_saturation_variant():
    """Half the static output scale: the largest outputs must saturate to 448 (0x7E)."""
    wl = workloads.workload(4, m=256, n=256, k=512, out_scale=0.5)
    inp = workloads.generate(wl)
    ref, u = fp8_reference(inp, np.arange(wl.m))
    assert np.any(ref == 0x7E)
    L = layers().make_layer(inp, with_unfused=False)
    case(f"fp8_fused saturation {wl}")
    y = L.forward()
    torch.cuda.synchronize()
    got = host(y, "fp8")
    assert_codes_within_one(got, ref)
    assert np.all(got[u / inp["s_y"] >= 464.0] == 0x7E)


# ---------------------------------------------------------------------------
# The e4m3 quantiser: bit-exact against the oracle on identical fp32 inputs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("inv", [1.0, 0.125, float(np.float32(1 / 3.7)), float(np.float32(1 / 11.3))])
def test_quantiser_bit_exact_exhaustive(inv):
    """Every fp32 pattern whose scaled value falls in [2^-12, 512) (about 21 binades x 2^23),
    plus samples of the saturating, underflowing and negative ranges."""
    d = dlf()
    lo = np.float32(2.0 ** -12 / inv).view(np.uint32)
    hi = np.float32(512.0 / inv).view(np.uint32)
    step = 1 << 24
    codes = torch.empty(step, dtype=torch.uint8, device="cuda")
    case(f"quant exhaustive inv={inv} patterns={int(hi) - int(lo)}")
    for start in range(int(lo), int(hi), step):
        n = min(step, int(hi) - start)
        bits = torch.arange(start, start + n, dtype=torch.int64, device="cuda").to(torch.int32)
        v = bits.view(torch.float32)
        d.dlf_quant_apply(n, v, inv, codes[:n])
        got = codes[:n].cpu().numpy()
        ref = oracle.quant_f32(v.cpu().numpy(), inv)
        bad = np.nonzero(got != ref)[0]
        assert bad.size == 0, (start, v.cpu().numpy()[bad[:4]], got[bad[:4]], ref[bad[:4]])
    rng = np.random.default_rng(1)
    extra = np.concatenate([
        rng.uniform(0, 2.0 ** -12 / inv, 100000), rng.uniform(448 / inv, 1e6 / inv, 100000),
        -rng.uniform(0, 600 / inv, 200000), [0.0, -0.0, 448 / inv, 464 / inv, 3e38],
    ]).astype(np.float32)
    vt = torch.from_numpy(extra).cuda()
    out = torch.empty(extra.size, dtype=torch.uint8, device="cuda")
    d.dlf_quant_apply(extra.size, vt, inv, out)
    np.testing.assert_array_equal(out.cpu().numpy(), oracle.quant_f32(extra, inv))


# ---------------------------------------------------------------------------
# Elementwise passes of the unfused chain (odd sizes exercise the scalar tails)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_unfused_eltwise_passes(dt):
    d = dlf()
    rng = np.random.default_rng(5)
    rows, c = 1001, 24
    y32 = rng.standard_normal((rows, c)).astype(np.float32)
    r32 = rng.standard_normal((rows, c)).astype(np.float32)
    store = (lambda a: a) if dt == "f32" else workloads.bf16_bits
    y_s, r_s = store(y32), store(r32)
    L = layers()
    y, r = L.to_device(y_s, dt), L.to_device(r_s, dt)
    g, b, mu = rng.uniform(0.5, 1.5, c), rng.normal(0, 0.1, c), rng.normal(0, 0.1, c)
    var = rng.uniform(1e-3, 1, c)
    P = [torch.from_numpy(np.asarray(a, np.float32)).cuda() for a in (g, b, mu, var)]
    out = torch.empty_like(y)
    tol = TOL[dt]
    yw, rw = oracle.widen(y_s, dt), oracle.widen(r_s, dt)
    P32 = [np.asarray(a, np.float32) for a in (g, b, mu, var)]
    case(f"bn_apply {dt}")
    d.dlf_bn_apply(rows, c, dt, y, *P, 1e-5, out)
    torch.cuda.synchronize()
    assert oracle.rel_error(oracle.widen(host(out, dt), dt), oracle.batchnorm(yw, *P32, 1e-5)) <= tol
    case(f"scale_shift {dt}")
    d.dlf_scale_shift_apply(rows, c, dt, y, P[0], P[1], out)
    torch.cuda.synchronize()
    ref = yw * P32[0].astype(np.float64) + P32[1].astype(np.float64)
    assert oracle.rel_error(oracle.widen(host(out, dt), dt), ref) <= tol
    case(f"add {dt}")
    d.dlf_add(rows * c - 3, dt, y, r, out)
    torch.cuda.synchronize()
    got = oracle.widen(host(out, dt), dt).ravel()[:rows * c - 3]
    assert oracle.rel_error(got, oracle.add(yw, rw).ravel()[:rows * c - 3]) <= tol
    for act in ("relu", "gelu_tanh", "gelu_erf"):
        case(f"act {act} {dt}")
        d.dlf_act_apply(rows * c - 5, dt, act, y, out)
        torch.cuda.synchronize()
        got = oracle.widen(host(out, dt), dt).ravel()[:rows * c - 5]
        assert oracle.rel_error(got, oracle.activation(yw, act).ravel()[:rows * c - 5]) <= tol


# ---------------------------------------------------------------------------
# Networks under the host fusion pass
# ---------------------------------------------------------------------------
NETWORKS = [
    # the benchmarked stage's widths and resolution (56x56x256 -> 28x28x512), 4 of its 32 images
    ("stage", dict(n=4, h=56, w=56, cin=256, cmid=128, cout=512, stride=2, blocks=2)),
    ("stage", dict(n=2, h=14, w=14, cin=64, cmid=32, cout=128, stride=2, blocks=2)),
    ("stage", dict(n=3, h=9, w=11, cin=24, cmid=16, cout=40, stride=2, blocks=3)),
    ("stem", dict(n=2, h=32, w=32)),
    ("stem", dict(n=2, h=32, w=30)),
]


@pytest.mark.parametrize("fuse", [True, False])
@pytest.mark.parametrize("i", range(len(NETWORKS)))
def test_network_under_the_fusion_plan(i, fuse):
    """The library's plan (identical to the oracle's) executed through the C ABI, checked layer
    by layer: every tensor the plan keeps in memory against the oracle's plain definition of the
    step that writes it (a fused chain: conv with the master weights -> BN -> [+ residual] ->
    activation, unfolded; any other op on its own), evaluated in binary64 on the GPU's own stored
    input tensors.  Each step is one fused launch or one unfused op, so each is held to the
    single-layer bf16 bar, with the floor of the metric taken per channel before the step's
    activation (the activation follows every rounding of the method; with batch statistics
    that do not centre a channel, ReLU leaves some channels nearly empty, and their rms after
    it says nothing about the size of the rounding).  The end-to-end difference to the oracle network (every step on the
    oracle's own stored tensors) is printed as a report: it adds the steps' differences along
    the path and is no parity bar."""
    from oracle import fusion as ofusion, network as onet
    from workloads import graphs
    from dl_fusion_amd.network import Network
    kind, kw = NETWORKS[i]
    g = graphs.resnet_stage_graph(**kw) if kind == "stage" else graphs.stem_graph(**kw)
    params = graphs.draw_params(g, seed=7 + i)
    case(f"network {kind} {kw} fuse={fuse}")
    net = Network(g, params, fuse=fuse)
    plan = ofusion.plan(g, net_ridge(), net_frac()) if fuse else []
    assert [p["nodes"] for p in net.plan] == [p["nodes"] for p in plan]
    bits = {j: workloads.bf16_bits(params[j]["x"]) for j in net.inputs}
    dev = {j: layers().to_device(b, "bf16") for j, b in bits.items()}
    net.forward(dev)
    torch.cuda.synchronize()
    steps = onet.steps(g, plan)
    assert sorted(net.bufs) == sorted(steps)
    stored = {j: oracle.widen(b, "bf16") for j, b in bits.items()}
    stored.update({j: oracle.widen(host(t, "bf16"), "bf16") for j, t in net.bufs.items()})
    for j, nodes in steps.items():
        pre, ref = onet.step(g, params, stored, nodes, with_pre=True)
        err = oracle.rel_error(stored[j], ref, floor_of=pre)
        assert err <= TOL["bf16"], (j, [g[k]["op"] for k in nodes], err)
    ref_net = onet.forward(g, params, bits, plan)
    end = max(oracle.rel_error(stored[j], ref_net[j]) for j in net.outputs)
    print(f"[report] network {kind} fuse={fuse}: end-to-end rel error {end:.3e} over "
          f"{len(steps)} stored tensors", flush=True)
    if fuse:
        assert net.launches == len(plan) + sum(
            1 for j, nd in enumerate(g) if nd["op"] != "input" and all(j not in p["nodes"] for p in plan))


def net_ridge():
    from dl_fusion_amd.network import RIDGE_BF16
    return RIDGE_BF16


def net_frac():
    from dl_fusion_amd.network import OVERHEAD_FRAC
    return OVERHEAD_FRAC


# ---------------------------------------------------------------------------
# Feed-forward block in one kernel
# ---------------------------------------------------------------------------
FFN_CASES = [
    dict(m=37, d_model=768, d_ff=3072, act="gelu_tanh", residual=True),
    dict(m=1, d_model=256, d_ff=256, act="relu", residual=False),
    dict(m=100, d_model=512, d_ff=1024, act="gelu_erf", residual=True),
    dict(m=64, d_model=1024, d_ff=512, act="none", residual=False),
    dict(m=250, d_model=768, d_ff=768, act="relu", residual=True),
]


@pytest.mark.parametrize("i", range(len(FFN_CASES)))
def test_ffn_fused_against_oracle(i):
    wl = workloads.FfnWorkload(f"ffn{i}", seed=50 + i, **FFN_CASES[i])
    inp = workloads.generate(wl)
    ref = oracle.ffn(inp)
    L = layers().make_layer(inp, with_unfused=(i < 2))
    case(f"ffn fused {wl}")
    buf, y = guarded((wl.m, wl.d_model), torch.bfloat16)
    L.forward(y=y)
    torch.cuda.synchronize()
    assert guard_intact(buf, y.numel())
    # with a handful of tokens the per-column floor of the metric degenerates to the element
    # itself (a cancelled output is then judged on its own rounding); the floor is then the
    # rms over each token's whole output row
    metric = oracle.rel_error if wl.m >= 8 else (lambda g, o: oracle.rel_error(g.reshape(-1), o.reshape(-1)))
    err = metric(oracle.widen(host(y, "bf16"), "bf16"), ref)
    assert err <= TOL["bf16"], err
    if i < 2:
        case(f"ffn unfused {wl}")
        yu = L.forward_unfused()
        torch.cuda.synchronize()
        err = metric(oracle.widen(host(yu, "bf16"), "bf16"), ref)
        assert err <= TOL["bf16"], ("unfused", err)


@pytest.mark.parametrize("tok", ["32", "64"])
def test_ffn_token_blocks(tok):
    """Both workgroup sizes (32 and 64 tokens) on ragged token counts, forced."""
    for i, kw in enumerate([dict(m=150, d_model=768, d_ff=512, act="gelu_tanh", residual=True),
                            dict(m=65, d_model=256, d_ff=768, act="relu", residual=False),
                            dict(m=64, d_model=512, d_ff=256, act="gelu_erf", residual=True)]):
        wl = workloads.FfnWorkload(f"ffn_tok{tok}_{i}", seed=70 + i, **kw)
        inp = workloads.generate(wl)
        ref = oracle.ffn(inp)
        L = layers().make_layer(inp, with_unfused=False)
        case(f"ffn fused tok={tok} {wl}")
        ENV["DLF_FFN_TOK"] = tok
        try:
            buf, y = guarded((wl.m, wl.d_model), torch.bfloat16)
            L.forward(y=y)
            torch.cuda.synchronize()
        finally:
            ENV.pop("DLF_FFN_TOK", None)
        assert guard_intact(buf, y.numel())
        err = oracle.rel_error(oracle.widen(host(y, "bf16"), "bf16"), ref)
        assert err <= TOL["bf16"], (tok, i, err)


def test_ffn_bert_base_full_size_sampled():
    """BERT-base's block at 8192 tokens: 256 sampled tokens (first and last among them)."""
    wl = workloads.FFN_BERT_BASE
    inp = workloads.generate(wl)
    L = layers().make_layer(inp, with_unfused=False)
    case(f"ffn fused {wl}")
    y = L.forward()
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, wl.m - 1], np.random.default_rng(6).integers(0, wl.m, 254)]))
    ref = oracle.ffn(inp, rows=rows)
    got = oracle.widen(host(y, "bf16"), "bf16")[rows]
    err = oracle.rel_error(got, ref)
    assert err <= TOL["bf16"], err


def test_ffn_without_biases():
    wl = workloads.FfnWorkload("ffn_nobias", m=40, d_model=256, d_ff=512, act="gelu_tanh", residual=False, seed=61)
    inp = workloads.generate(wl)
    inp["b1"] = np.zeros_like(inp["b1"])
    inp["b2"] = np.zeros_like(inp["b2"])
    ref = oracle.ffn(inp)
    d = dlf()
    L = layers().make_layer(inp, with_unfused=False)
    case("ffn without biases")
    d.dlf_ffn_fused(L.desc, L.x, L.w1p, None, L.w2p, None, None, L.y)
    torch.cuda.synchronize()
    err = oracle.rel_error(oracle.widen(host(L.y, "bf16"), "bf16"), ref)
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("split", ["2", "3", "0", "auto"])
def test_ffn_split_over_d_ff(split):
    """The d_ff split (S workgroups a token block, fp32 partial sums through the workspace, a
    second kernel adding them with b2 and the residual): forced to 2 and 3 parts, off
    (DLF_FFN_SPLIT), and the library's own choice (as many parts as fit 256 workgroups, at
    most one a chunk), on ragged token counts, every d_model it is built for and chunk counts that do
    not divide evenly; the workspace has a guard band.  The third case has no biases.  Unsplit,
    the 64-token workgroup is forced (DLF_FFN_TOK), so its walk over several d_ff chunks (the
    single h buffer behind a second barrier) runs on ragged token tails at d_model 256, 512 and
    768."""
    cases = [dict(m=150, d_model=768, d_ff=768, act="gelu_tanh", residual=True),
             dict(m=200, d_model=256, d_ff=1024, act="relu", residual=False),
             dict(m=300, d_model=512, d_ff=1280, act="gelu_erf", residual=True)]
    d = dlf()
    if split == "0":
        ENV["DLF_FFN_TOK"] = "64"
    if split != "auto":
        ENV["DLF_FFN_SPLIT"] = split
    try:
        for i, kw in enumerate(cases):
            wl = workloads.FfnWorkload(f"ffn_split{split}_{i}", seed=80 + i, **kw)
            nchunks = wl.d_ff // 256
            parts = {"0": 1, "auto": min(256 // -(-wl.m // 32), nchunks)}.get(split) or min(int(split), nchunks)
            inp = workloads.generate(wl)
            if i == 2:
                inp["b1"] = np.zeros_like(inp["b1"])
                inp["b2"] = np.zeros_like(inp["b2"])
            ref = oracle.ffn(inp)
            L = layers().make_layer(inp, with_unfused=False)
            assert L.ws_bytes == (parts * wl.m * wl.d_model * 4 if parts > 1 else 0), (L.ws_bytes, parts)
            wbuf, ws = guarded((max(L.ws_bytes, 16),), torch.uint8)
            case(f"ffn fused split={split} parts={parts} {wl}")
            buf, y = guarded((wl.m, wl.d_model), torch.bfloat16)
            if i == 2:
                d.dlf_ffn_fused_ws(L.desc, L.x, L.w1p, None, L.w2p, None, L.res, y, ws, L.ws_bytes)
            else:
                d.dlf_ffn_fused_ws(L.desc, L.x, L.w1p, L.b1, L.w2p, L.b2, L.res, y, ws, L.ws_bytes)
            torch.cuda.synchronize()
            assert guard_intact(buf, y.numel())
            assert guard_intact(wbuf, ws.numel()), "write beyond the workspace"
            err = oracle.rel_error(oracle.widen(host(y, "bf16"), "bf16"), ref)
            assert err <= TOL["bf16"], (split, i, err)
    finally:
        ENV.pop("DLF_FFN_SPLIT", None)
        ENV.pop("DLF_FFN_TOK", None)
