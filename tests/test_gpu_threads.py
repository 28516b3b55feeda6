"""Calls from several host threads at once, each on its own stream: the library keeps no
per-call global state (the CU-count cache is written once with the same value), so every
thread's results equal those of the same calls made one after another.  ctypes releases
the GIL during each library call, so the launches of different threads interleave."""
import threading

import pytest
import torch

import fp8_fine_grained_fp8q_amd as fq

pytestmark = pytest.mark.gpu

THREADS = 4
M, N, K = 512, 1024, 1024
G, GN = 4, 512


def _randn(shape, seed, scale=1.0):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return (torch.randn(shape, device="cuda", generator=g) * scale).to(torch.bfloat16)


def _inputs(i):
    x = _randn((M, K), 100 + i)
    w = _randn((N, K), 200 + i, 0.02)
    we = _randn((G, GN, K), 300 + i, 0.02)
    sizes = torch.tensor([0, 97 + 13 * i, 128, 200 - 7 * i], dtype=torch.int64)
    offsets = torch.zeros(G + 1, dtype=torch.int32)
    offsets[1:] = torch.cumsum(sizes, 0).to(torch.int32)
    return x, w, we, offsets.cuda()


def _step(x, w, we, offsets, outs, stream):
    """Both quantizers, the dense GEMM, the expert-weight quantizer and the grouped GEMM on
    the first offsets[-1] rows of x, all on `stream`, into the preallocated outs."""
    xq, sa, wq, sb, c, weq, web, yg = outs
    fq.fp8q_quantize_act_w(x, w, xq=xq, sa=sa, wq=wq, sb=sb, stream=stream)
    fq.fp8q_gemm_blockscaled(xq, sa, wq, sb, out=c, stream=stream)
    fq.fp8q_quantize_w_128x128(we, wq=weq, sb=web, stream=stream)
    fq.fp8q_grouped_gemm_blockscaled(xq, sa, weq, web, offsets, out=yg, stream=stream)


def _outs():
    dev = "cuda"
    return (torch.empty((M, K), dtype=torch.uint8, device=dev), torch.empty((K // 128, M), device=dev),
            torch.empty((N, K), dtype=torch.uint8, device=dev), torch.empty((N // 128, K // 128), device=dev),
            torch.empty((M, N), dtype=torch.bfloat16, device=dev),
            torch.empty((G, GN, K), dtype=torch.uint8, device=dev),
            torch.empty((G, GN // 128, K // 128), device=dev),
            torch.zeros((M, GN), dtype=torch.bfloat16, device=dev))


def test_threads_on_their_own_streams_match_serial_calls():
    inputs = [_inputs(i) for i in range(THREADS)]
    ref = []
    for i in range(THREADS):
        o = _outs()
        _step(*inputs[i], o, torch.cuda.current_stream())
        ref.append(o)
    torch.cuda.synchronize()

    outs = [_outs() for _ in range(THREADS)]
    streams = [torch.cuda.Stream() for _ in range(THREADS)]
    start = threading.Barrier(THREADS)
    errors = []

    def work(i):
        try:
            start.wait()
            for _ in range(3):
                _step(*inputs[i], outs[i], streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported below; a thread's exception would otherwise vanish
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(THREADS):
        rows = int(inputs[i][3][-1].item())
        for j, (a, b) in enumerate(zip(outs[i], ref[i])):
            if j == 7:
                a, b = a[:rows], b[:rows]
            if a.dtype in (torch.bfloat16, torch.float32):
                a = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32)
                b = b.view(a.dtype)
            assert torch.equal(a, b), f"thread {i}, output {j}"
