"""Graph replays of the fused kernels.

The benchmark times every workload as a captured HIP graph, so each kernel route must give,
replay after replay, exactly what its eager launch gives.  Each case captures three launches of
one layer into a graph and replays it three times.  Between replays, eager work runs: the output
is cleared by a fill kernel and an unrelated reduction is computed.  Every replay must match the
eager output bit for bit, since the kernels are deterministic.  The shapes are chosen so that
each case takes a different kernel of the library (the routing rules of dlf_conv_fused,
dlf_gemm_fused and dlf_ffn_fused_ws).
"""
import pytest

import workloads

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

CASES = {
    # Cin = 64, 3x3 stride 1: the persistent kernel with resident weights
    "conv_halo_res": lambda: workloads.workload(1, n=2, h=20, w=24),
    # 7x7 images, Cin % 64 == 0, N Cout / 32 >= 128: the whole-image kernel, with a residual
    "conv_halo_img": lambda: workloads.workload(2, n=32, h=7, w=7, cin=128, cout=128),
    # Cin = 128, a 28x28 image: the halo kernel with streamed weights
    "conv_halo_stream": lambda: workloads.workload(1, n=2, h=28, w=28, cin=128, cout=128),
    # fp32, K = 144: the fp32 kernel with its weights staged in LDS
    "conv_f32": lambda: workloads.workload(0),
    # c_in = 3, 7x7 stride 2: the small-channel kernel with compute and store waves
    "conv_small_channel": lambda: workloads.workload(1, n=2, h=64, w=64, cin=3, cout=64, kh=7, kw=7, stride=2,
                                                       pad=3),
    # a 3x3 stride-2 layer: the implicit GEMM
    "conv_implicit_gemm": lambda: workloads.workload(1, n=2, h=16, w=16, cin=32, cout=64, stride=2),
    # 4096 x 4096 outputs: the sixteen-wave 256 x 256 tile
    "gemm_256x256": lambda: workloads.GemmWorkload("gemm_4096x4096x512", 4096, 4096, 512),
    # K = 256, 16384 x 256 outputs: the streaming GEMM
    "gemm_streaming": lambda: workloads.GemmWorkload("gemm_16384x256x256", 16384, 256, 256, act="relu"),
    "gemm_fp8_quant": lambda: workloads.Fp8GemmWorkload("fp8_512x512x256", 512, 512, 256),
    # 512 tokens: the FFN block split over d_ff, partial sums through its workspace
    "ffn_split": lambda: workloads.FfnWorkload("ffn_512x768x1536", 512, 768, 1536),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dl_fusion_amd  # noqa: F401  (loud failure if the library is missing)
    torch.cuda.set_device(0)


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_the_eager_launch(name):
    from dl_fusion_amd import layers
    print(f"graph replay case: {name}", flush=True)
    layer = layers.make_layer(workloads.generate(CASES[name]()), with_unfused=False)
    out = layer.forward()
    torch.cuda.synchronize()
    ref = out.clone()
    if getattr(layer, "ws_bytes", 0):
        print(f"  workspace {layer.ws_bytes} bytes", flush=True)

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for _ in range(3):
                layer.forward()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    other = torch.randn(1 << 20, device="cuda")
    for r in range(3):
        out.zero_()
        float(other.sum())                     # eager work and a synchronisation between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{name}: replay {r} differs from the eager launch"
