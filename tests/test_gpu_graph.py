"""The entry points under HIP graph capture: they issue only kernel launches on the caller's
stream (no allocation, no memset, no synchronization on the default path), so a captured
step replays the same kernels.  Each graph is replayed several times with new input values
copied into its static inputs, eager work and synchronizations between the replays, and
every replay is compared bit for bit with an eager run of the same calls on the same
inputs (the eager path itself is checked against the oracle by the other GPU tests)."""
import pytest
import torch

import fp8_fine_grained_fp8q_amd as fq

pytestmark = pytest.mark.gpu


def _randn(shape, seed, scale=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, device="cuda", generator=g) * scale).to(torch.bfloat16)


def _same(a, b, what):
    if a.dtype in (torch.bfloat16, torch.float32):
        a = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32)
        b = b.view(a.dtype)
    assert torch.equal(a, b), what


@pytest.mark.parametrize("M,N,K", [(1024, 2048, 1024), (3072, 4096, 512)])
def test_dense_step_graph_replays_match_eager(M, N, K):
    """Both quantizers in one launch, then the block-scaled GEMM (BF16 out), captured once.
    (3072, 4096, 512) takes the two-region tile plan, (1024, 2048, 1024) the uniform one."""
    x = _randn((M, K), 1)
    w = _randn((N, K), 2, 0.02)
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((K // 128, M), dtype=torch.float32, device="cuda")
    wq = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    sb = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        fq.fp8q_quantize_act_w(x, w, xq=xq, sa=sa, wq=wq, sb=sb)
        fq.fp8q_gemm_blockscaled(xq, sa, wq, sb, out=c)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    for rep in range(4):
        x.copy_(_randn((M, K), 10 + rep))
        w.copy_(_randn((N, K), 20 + rep, 0.02))
        rq, rs, rwq, rsb = fq.fp8q_quantize_act_w(x, w)
        rc = fq.fp8q_gemm_blockscaled(rq, rs, rwq, rsb)
        _ = fq.fp8q_quantize_act_1x128(_randn((256, K), 30 + rep))  # unrelated eager work
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(xq, rq, f"replay {rep}: activation codes")
        _same(sa, rs, f"replay {rep}: activation scales")
        _same(wq, rwq, f"replay {rep}: weight codes")
        _same(sb, rsb, f"replay {rep}: weight scales")
        _same(c, rc, f"replay {rep}: GEMM output")


def test_moe_chain_graph_replays_match_eager():
    """Quantize the tokens, dispatch them to 16 local experts (of 64, top 4), the grouped
    GEMM over the dispatched rows (FP32 out), and the gated combine, captured once; the
    routing changes between replays, so the expert sizes do too."""
    T, K, N, E, G, k = 512, 1024, 512, 64, 16, 4
    x = _randn((T, K), 3)
    wexp = _randn((G, N, K), 4, 0.02)
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    gate = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    wq, sb = fq.fp8q_quantize_w_128x128(wexp)

    def routing(seed):
        g = torch.Generator(device="cuda").manual_seed(seed)
        scores = torch.rand((T, E), device="cuda", generator=g)
        top = torch.topk(scores, k, dim=1)
        return top.indices.to(torch.int32), top.values / top.values.sum(dim=1, keepdim=True)

    def chain():
        xq, sa = fq.fp8q_quantize_act_1x128(x)
        xs, ss, offsets, token_row, _ = fq.fp8q_moe_dispatch(ids, xq, sa, 0, G)
        ys = fq.fp8q_grouped_gemm_blockscaled(xs, ss, wq, sb, offsets, out_dtype=torch.float32)
        y = fq.fp8q_moe_combine(ys, token_row, gate, out_dtype=torch.float32)
        return offsets, token_row, ys, y

    i0, g0 = routing(100)
    ids.copy_(i0)
    gate.copy_(g0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        chain()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = chain()

    for rep in range(4):
        x.copy_(_randn((T, K), 40 + rep))
        i, gw = routing(200 + rep)
        ids.copy_(i)
        gate.copy_(gw)
        ref = chain()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        offsets, token_row, ys, y = outs
        _same(offsets, ref[0], f"replay {rep}: offsets")
        _same(token_row, ref[1], f"replay {rep}: token rows")
        rows = int(offsets[-1].item())
        assert rows > 0
        _same(ys[:rows], ref[2][:rows], f"replay {rep}: grouped GEMM output")
        _same(y, ref[3], f"replay {rep}: combined output")
