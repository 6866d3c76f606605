"""The no-allocation FFN entry point (dlf_ffn_fused_noalloc) against the workspace one.

dlf_ffn_fused_noalloc runs the same kernels as dlf_ffn_fused_ws with the d_ff split's partial
sums in the library's static device scratch instead of a caller's workspace, so its output must
equal the workspace entry point's bit for bit, and the oracle's within the bf16 bar.  Two calls
in a row, the second on a smaller block (the scratch keeps the first call's partial sums), then
a block that needs no scratch, and a block whose split would need more scratch than the array
holds: rejected before anything is launched.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

GUARD = 4096
CASES = [
    # 1000 tokens: 32 blocks of 32 split into 8 parts, 24.6 MB of partial sums
    dict(m=1000, d_model=768, d_ff=3072, act="gelu_tanh", residual=True),
    # then a smaller one: 5 blocks, 5 parts over a ragged token tail, 1.5 MB
    dict(m=150, d_model=512, d_ff=1280, act="gelu_erf", residual=False),
    # d_model 1024 is never split: no scratch at all
    dict(m=100, d_model=1024, d_ff=512, act="relu", residual=True),
]


def guarded_bf16(shape):
    n = int(np.prod(shape))
    buf = torch.empty(n + GUARD, dtype=torch.bfloat16, device="cuda")
    buf.view(torch.int16).fill_(0x7FA5)
    return buf, buf[:n].view(shape)


def intact(buf, n):
    return bool((buf[n:].view(torch.int16) == 0x7FA5).all())


def test_ffn_noalloc_matches_the_workspace_entry_point():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dl_fusion_amd as d
    from dl_fusion_amd.layers import make_layer, to_host
    torch.cuda.set_device(0)
    for i, kw in enumerate(CASES):
        wl = workloads.FfnWorkload(f"ffn_noalloc_{i}", seed=90 + i, **kw)
        inp = workloads.generate(wl)
        L = make_layer(inp, with_unfused=False)
        print(f"\n[case] noalloc {wl} workspace={L.ws_bytes}", flush=True)
        assert L.ws_bytes <= d.DLF_FFN_NOALLOC_SCRATCH_BYTES
        assert (L.ws_bytes > 0) == (i < 2)
        _, y_ws = guarded_bf16((wl.m, wl.d_model))
        d.dlf_ffn_fused_ws(L.desc, L.x, L.w1p, L.b1, L.w2p, L.b2, L.res, y_ws, L.ws, L.ws_bytes)
        buf, y = guarded_bf16((wl.m, wl.d_model))
        d.dlf_ffn_fused_noalloc(L.desc, L.x, L.w1p, L.b1, L.w2p, L.b2, L.res, y)
        torch.cuda.synchronize()
        assert intact(buf, y.numel()), "store beyond the output"
        assert torch.equal(y.view(torch.int16), y_ws.view(torch.int16)), i
        err = oracle.rel_error(oracle.widen(to_host(y, "bf16"), "bf16"), oracle.ffn(inp))
        assert err <= 2e-2, (i, err)
        del L


def test_ffn_noalloc_rejects_a_split_beyond_its_scratch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dl_fusion_amd as d
    torch.cuda.set_device(0)
    # 4096 tokens of d_model 768: 64 blocks of 64 in 4 parts, 50 MB of partial sums
    m, dm, dff = 4096, 768, 3072
    desc = d.ffn_desc(m, dm, dff, "gelu_tanh")
    assert d.dlf_ffn_workspace_bytes(desc) > d.DLF_FFN_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((m, dm), dtype=torch.bfloat16, device="cuda")
    w1 = torch.zeros((dff, dm), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((dm, dff), dtype=torch.bfloat16, device="cuda")
    buf, y = guarded_bf16((m, dm))
    y.view(torch.int16).fill_(0x1234)
    with pytest.raises(d.DlfError) as e:
        d.dlf_ffn_fused_noalloc(desc, x, w1, None, w2, None, None, y)
    assert e.value.status == d.DLF_ERR_INVALID_ARG and "scratch" in e.value.detail
    torch.cuda.synchronize()
    assert bool((y.view(torch.int16) == 0x1234).all()) and intact(buf, y.numel()), "a rejected call wrote"
