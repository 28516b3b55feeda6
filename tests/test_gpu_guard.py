"""Guard bands around every output: each entry point is called through the C ABI with its
outputs placed inside larger buffers filled with a sentinel byte, on ragged shapes (rows
not a multiple of the tile height, an empty expert, a short final chunk); the sentinel
bytes before and after every output must be untouched afterwards.  Catches writes past
the end (or before the start) of an output that the value checks elsewhere cannot see."""
import ctypes

import numpy as np
import pytest
import torch

import fp8_fine_grained_fp8q_amd as fq

pytestmark = pytest.mark.gpu

GUARD = 4096      # bytes on either side; keeps every output 16-byte aligned
SENTINEL = 0xA5


class Guarded:
    """An output tensor of `shape`/`dtype` inside a sentinel-filled byte buffer."""

    def __init__(self, shape, dtype):
        itemsize = torch.empty((), dtype=dtype).element_size()
        self.n = int(np.prod(shape)) * itemsize
        self.raw = torch.full((self.n + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD:GUARD + self.n].view(dtype).view(shape)

    @property
    def ptr(self):
        return ctypes.c_void_p(self.t.data_ptr())

    def intact(self):
        h = self.raw.cpu().numpy()
        return bool(np.all(h[:GUARD] == SENTINEL) and np.all(h[GUARD + self.n:] == SENTINEL))


def p(t):
    return ctypes.c_void_p(t.data_ptr())


def bf16(*shape, seed=0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(*shape, device="cuda", generator=g).to(torch.bfloat16)


def run(name, *args):
    lib = fq.load_library()
    rc = getattr(lib, name)(*args, None)
    torch.cuda.synchronize()
    assert rc == 0, f"{name} returned {rc}"


def assert_intact(*outs):
    for i, o in enumerate(outs):
        assert o.intact(), f"output {i} written outside its range"


def codes(M, K, seed):
    xq, sa = fq.fp8q_quantize_act_1x128(bf16(M, K, seed=seed))
    return xq, sa


def test_quantizers_guarded():
    M, K, G, N = 300, 384, 2, 256
    x, w = bf16(M, K, seed=1), bf16(G, N, K, seed=2)
    xq, sa = Guarded((M, K), torch.uint8), Guarded((K // 128, M), torch.float32)
    run("fp8q_quantize_act_1x128", p(x), M, K, xq.ptr, sa.ptr)
    assert_intact(xq, sa)
    wq, sb = Guarded((G, N, K), torch.uint8), Guarded((G, N // 128, K // 128), torch.float32)
    run("fp8q_quantize_w_128x128", p(w), G, N, K, wq.ptr, sb.ptr)
    assert_intact(wq, sb)
    wq, sb = Guarded((G, N, K), torch.uint8), Guarded((G, N // 128, K // 128), torch.float32)
    wqt, sbt = Guarded((G, K, N), torch.uint8), Guarded((G, K // 128, N // 128), torch.float32)
    run("fp8q_quantize_w_128x128_t", p(w), G, N, K, wq.ptr, sb.ptr, wqt.ptr, sbt.ptr)
    assert_intact(wq, sb, wqt, sbt)
    xq, sa = Guarded((M, K), torch.uint8), Guarded((K // 128, M), torch.float32)
    wq, sb = Guarded((G, N, K), torch.uint8), Guarded((G, N // 128, K // 128), torch.float32)
    run("fp8q_quantize_act_w", p(x), M, p(w), G, N, K, xq.ptr, sa.ptr, wq.ptr, sb.ptr)
    assert_intact(xq, sa, wq, sb)
    Md = 256
    xd = bf16(Md, K, seed=3)
    xq, sa = Guarded((Md, K), torch.uint8), Guarded((K // 128, Md), torch.float32)
    xqt, sat = Guarded((K, Md), torch.uint8), Guarded((Md // 128, K), torch.float32)
    run("fp8q_quantize_act_dual", p(xd), Md, K, xq.ptr, sa.ptr, xqt.ptr, sat.ptr)
    assert_intact(xq, sa, xqt, sat)
    I = 256
    gu = bf16(M, 2 * I, seed=4)
    hq, sh = Guarded((M, I), torch.uint8), Guarded((I // 128, M), torch.float32)
    run("fp8q_swiglu_quantize_act_1x128", p(gu), M, I, hq.ptr, sh.ptr)
    assert_intact(hq, sh)
    q, stats = Guarded((M * K,), torch.uint8), Guarded((3,), torch.int32)
    run("fp8q_quantize_per_tensor", p(x), M * K, None, q.ptr, stats.ptr)
    assert_intact(q, stats)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_gemms_guarded(out_dtype):
    code = fq.FP8Q_OUT_F32 if out_dtype == torch.float32 else fq.FP8Q_OUT_BF16
    M, N, K = 300, 384, 384
    xq, sa = codes(M, K, 5)
    wq, sb = fq.fp8q_quantize_w_128x128(bf16(N, K, seed=6))
    c = Guarded((M, N), out_dtype)
    run("fp8q_gemm_blockscaled", p(xq), p(sa), p(wq), p(sb), M, N, K, c.ptr, code)
    assert_intact(c)
    # row-scaled: both operands with 1x128 row scales
    bq, sbr = codes(N, K, 7)
    c = Guarded((M, N), out_dtype)
    run("fp8q_gemm_rowscaled", p(xq), p(sa), p(bq), p(sbr), M, N, K, c.ptr, code)
    assert_intact(c)
    # grouped, with an empty expert
    G = 3
    wg, sbg = fq.fp8q_quantize_w_128x128(bf16(G, N, K, seed=8))
    offsets = torch.tensor([0, 100, 100, M], dtype=torch.int32, device="cuda")
    c = Guarded((M, N), out_dtype)
    run("fp8q_grouped_gemm_blockscaled", p(xq), p(sa), p(wg), p(sbg), p(offsets), G, M, N, K, c.ptr, code)
    assert_intact(c)


def test_dispatch_and_combine_guarded():
    T, k, E, K, N = 300, 4, 8, 256, 264
    ids = torch.randint(0, 16, (T, k), dtype=torch.int32, device="cuda")
    xq, sa = codes(T, K, 9)
    for cap in (T * k, 500):   # room for every routed pair, and a short capacity
        xs, ss = Guarded((cap, K), torch.uint8), Guarded((K // 128, cap), torch.float32)
        off, tr = Guarded((E + 1,), torch.int32), Guarded((T, k), torch.int32)
        rt = Guarded((cap,), torch.int32)
        run("fp8q_moe_dispatch", p(ids), T, k, 0, E, p(xq), p(sa), K, cap, xs.ptr, ss.ptr, off.ptr, tr.ptr, rt.ptr)
        assert_intact(xs, ss, off, tr, rt)
    out = torch.randn(T * k, N, device="cuda").to(torch.bfloat16)
    w = torch.rand(T, k, device="cuda")
    y = Guarded((T, N), torch.bfloat16)
    run("fp8q_moe_combine", p(out), fq.FP8Q_OUT_BF16, T * k, N, p(tr.t), p(w), T, k, y.ptr,
        fq.FP8Q_OUT_BF16)
    assert_intact(y)
    # a long routing (several chunks of the counting pass) and the FP32 combine
    T2 = 3000
    ids2 = torch.randint(0, 16, (T2, k), dtype=torch.int32, device="cuda")
    xq2, sa2 = codes(T2, K, 10)
    cap2 = T2 * k
    xs, ss = Guarded((cap2, K), torch.uint8), Guarded((K // 128, cap2), torch.float32)
    off, tr = Guarded((E + 1,), torch.int32), Guarded((T2, k), torch.int32)
    rt = Guarded((cap2,), torch.int32)
    run("fp8q_moe_dispatch", p(ids2), T2, k, 0, E, p(xq2), p(sa2), K, cap2, xs.ptr, ss.ptr, off.ptr, tr.ptr, rt.ptr)
    assert_intact(xs, ss, off, tr, rt)
    out2 = torch.randn(cap2, N, device="cuda")
    w2 = torch.rand(T2, k, device="cuda")
    y = Guarded((T2, N), torch.float32)
    run("fp8q_moe_combine", p(out2), fq.FP8Q_OUT_F32, cap2, N, p(tr.t), p(w2), T2, k, y.ptr, fq.FP8Q_OUT_F32)
    assert_intact(y)
