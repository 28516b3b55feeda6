"""GPU parity of the expert-parallel dispatch and combine against the oracle.

Dispatch: offsets, the (token, slot) -> row map, the row -> token map, and the packed codes
and scales are bit-exact (random routings with duplicate and non-local ids, k = 1..8,
empty cases, and the moe_layer workload at full size: 8192 tokens, top-8 of 256, 32 local
experts).  Combine: within the bound of its FP32 accumulation and output rounding (BF16
and FP32, expert outputs given as BF16 or FP32; synthetic expert outputs, full size too).
Also: the grouped GEMM on the dispatched rows equals the grouped GEMM on the moe_up
workload's host-sorted rows of the same tokens, bit for bit."""
import numpy as np
import pytest
import torch

import fp8_fine_grained_fp8q_amd as fq
import workloads as wl
from oracle import moe as om
from oracle import quant as oq

from helpers import dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def dispatch_both(x_u16, ids, e_begin, E):
    """GPU quantize + dispatch, and the oracle's; returns both result tuples (host arrays)."""
    xq, sa = fq.fp8q_quantize_act_1x128(dev_bf16(x_u16))
    xs, ss, off, tr, rt = fq.fp8q_moe_dispatch(dev(ids), xq, sa, e_begin, E)
    torch.cuda.synchronize()
    rq, rsa = oq.quantize_act_1x128(x_u16)
    roff, rrt, rtr = om.dispatch(ids, e_begin, E)
    pq, psa = om.pack(rq, rsa, rrt)
    return (host(xs), host(ss), host(off), host(tr), host(rt)), (pq, psa, roff, rtr, rrt)


def assert_dispatch_equal(got, ref):
    xs, ss, off, tr, rt = got
    pq, psa, roff, rtr, rrt = ref
    R = int(roff[-1])
    assert np.array_equal(off, roff), "offsets"
    assert np.array_equal(tr, rtr), "token -> row map"
    assert np.array_equal(rt[:R], rrt), "row -> token map"
    assert np.array_equal(xs[:R], pq), "packed codes"
    assert np.array_equal(ss[:, :R].view(np.uint32), psa.view(np.uint32)), "packed scales"


# The routing works in chunks of 1024 (token, slot) entries, the last taking the remainder
# (one chunk below 2048 entries): lone chunks, two chunks with a two-round tail, many chunks
# per scan thread (C > 1024 / E), E = 1024 (one scan thread per expert, 2 and 32 chunks), E = 1.
@pytest.mark.parametrize("T,k,E,e_begin,K,id_range", [(300, 8, 20, 16, 384, 64), (77, 1, 5, 0, 128, 64),
                                                      (129, 3, 64, 0, 256, 64), (64, 6, 1, 9, 128, 64),
                                                      (4100, 8, 512, 100, 128, 1024), (300, 8, 1024, 0, 128, 1500),
                                                      (2048, 1, 1, 3, 128, 8), (4096, 8, 1024, 0, 128, 2048)])
def test_dispatch_random(T, k, E, e_begin, K, id_range):
    rng = np.random.default_rng(T * 31 + k * 7 + E)
    x = wl.bf16_bits(rng.standard_normal((T, K), dtype=np.float32) * np.float32(4.0))
    ids = rng.integers(0, id_range, size=(T, k)).astype(np.int32)  # duplicates and non-local ids included
    got, ref = dispatch_both(x, ids, e_begin, E)
    assert_dispatch_equal(got, ref)


def test_dispatch_degenerate():
    x = wl.bf16_bits(np.ones((6, 128), np.float32))
    got, ref = dispatch_both(x, np.full((6, 2), 99, np.int32), 0, 32)      # nothing local
    assert_dispatch_equal(got, ref)
    assert int(got[2][-1]) == 0
    got, ref = dispatch_both(x, np.full((6, 1), 3, np.int32), 0, 8)        # every token to one expert
    assert_dispatch_equal(got, ref)
    xq = torch.empty((0, 128), dtype=torch.uint8, device="cuda")
    sa = torch.empty((1, 0), dtype=torch.float32, device="cuda")
    _, _, off, _, _ = fq.fp8q_moe_dispatch(torch.empty((0, 8), dtype=torch.int32, device="cuda"), xq, sa, 0, 4)
    torch.cuda.synchronize()
    assert host(off).tolist() == [0, 0, 0, 0, 0]


def test_dispatch_short_capacity():
    """A capacity below the routed count: the first `capacity` rows are as with room for
    all, the later ones are dropped (their slots read -1) and offsets still count them."""
    rng = np.random.default_rng(8)
    T, k, E, K = 200, 4, 16, 256
    x = wl.bf16_bits(rng.standard_normal((T, K), dtype=np.float32))
    ids = np.stack([rng.choice(32, k, replace=False) for _ in range(T)]).astype(np.int32)
    roff, rrt, rtr = om.dispatch(ids, 0, E)
    cap = int(roff[-1]) - 37
    xq, sa = fq.fp8q_quantize_act_1x128(dev_bf16(x))
    xs, ss, off, tr, rt = fq.fp8q_moe_dispatch(dev(ids), xq, sa, 0, E, capacity=cap)
    torch.cuda.synchronize()
    assert np.array_equal(host(off), roff)
    assert np.array_equal(host(tr), np.where(rtr < cap, rtr, -1))
    assert np.array_equal(host(rt), rrt[:cap])
    pq, psa = om.pack(*oq.quantize_act_1x128(x), rrt[:cap])
    assert np.array_equal(host(xs), pq) and np.array_equal(host(ss).view(np.uint32), psa.view(np.uint32))


def combine_check(out_d, token_row, w, out_dtype):
    """GPU combine of the expert outputs out_d (bf16 or float32 [capacity, N], CUDA) against
    the oracle's, within the bound of FP32 accumulation in slot order plus the output
    rounding."""
    y = fq.fp8q_moe_combine(out_d, dev(token_row), dev(w), out_dtype=out_dtype)
    torch.cuda.synchronize()
    R = int(token_row.max()) + 1 if token_row.size and token_row.max() >= 0 else 0
    used = host(out_d[:R]).astype(np.float64)  # the referenced rows, as the kernel saw them
    ref = om.combine(used, token_row, w)
    bound = om.combine_bound(used, token_row, w)
    k = token_row.shape[1]
    tol = ((2.0 ** -8 if out_dtype == torch.bfloat16 else 0.0) + k * 2.0 ** -23) * bound
    got = host(y).astype(np.float64)
    assert np.all(np.abs(got - ref) <= tol), f"combine off by {np.max(np.abs(got - ref) - tol)} beyond the bound"


@pytest.mark.parametrize("in_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_combine_random(in_dtype, out_dtype):
    rng = np.random.default_rng(11)
    T, k, R, N = 50, 8, 120, 264
    out = torch.from_numpy((rng.standard_normal((R, N)) * 3.0).astype(np.float32)).to(in_dtype).cuda()
    token_row = rng.integers(-1, R, size=(T, k)).astype(np.int32)
    token_row[3] = -1                       # a token with no local slot: y = 0
    w = rng.random((T, k)).astype(np.float32)
    combine_check(out, token_row, w, out_dtype)


def test_combine_skips_rows_past_capacity():
    """Slots whose row is at or past the expert outputs' row count (a dispatch that ran short
    of capacity leaves -1, but any row >= capacity) contribute nothing, as if not local."""
    rng = np.random.default_rng(13)
    T, k, R, N = 40, 4, 64, 136
    out = torch.from_numpy(rng.standard_normal((R, N)).astype(np.float32)).to(torch.bfloat16).cuda()
    token_row = rng.integers(-1, R + 30, size=(T, k)).astype(np.int32)   # some rows >= R
    w = rng.random((T, k)).astype(np.float32)
    y = fq.fp8q_moe_combine(out, dev(token_row), dev(w), out_dtype=torch.float32)
    torch.cuda.synchronize()
    kept = np.where(token_row < R, token_row, -1).astype(np.int32)
    used = host(out).astype(np.float64)
    ref = om.combine(used, kept, w)
    tol = k * 2.0 ** -23 * om.combine_bound(used, kept, w)
    assert np.all(np.abs(host(y).astype(np.float64) - ref) <= tol)


def test_moe_layer_full_size():
    """The moe_layer workload: 8192 tokens, top-8 of 256 experts, 32 local; dispatch
    bit-exact with the oracle, the same offsets as the workload's routing lists, the
    grouped up-projection on the dispatched rows identical to the one on the host-sorted
    moe_up rows, and the combine of synthetic expert outputs within its bound."""
    c = wl.moe_layer()
    ids, gate, x = c["topk_ids"], c["topk_w"], c["x"]
    got, ref = dispatch_both(x, ids, 0, 32)
    assert_dispatch_equal(got, ref)
    _, off_ref = wl.routing()
    assert np.array_equal(got[2], off_ref)

    # grouped GEMM on the dispatched rows == on the host-sorted rows of moe_up
    xq, sa = fq.fp8q_quantize_act_1x128(dev_bf16(x))
    xs, ss, off, tr, _ = fq.fp8q_moe_dispatch(dev(ids), xq, sa, 0, 32)
    wq, sb = fq.fp8q_quantize_w_128x128(dev_bf16(c["w"]))
    up = fq.fp8q_grouped_gemm_blockscaled(xs, ss, wq, sb, off)
    m = wl.moe_up()
    mq, msa = fq.fp8q_quantize_act_1x128(dev_bf16(m["x"]))
    up_ref = fq.fp8q_grouped_gemm_blockscaled(mq, msa, wq, sb, dev(m["offsets"]))
    torch.cuda.synchronize()
    R = int(host(off)[-1])
    assert torch.equal(up[:R].view(torch.int16), up_ref.view(torch.int16))

    # combine at full size with synthetic expert outputs (rows past R are never referenced)
    rng = np.random.default_rng(12)
    N = 7168
    out = torch.zeros((ids.size, N), dtype=torch.bfloat16, device="cuda")
    out[:R] = torch.from_numpy(rng.standard_normal((R, N), dtype=np.float32)).to(torch.bfloat16).cuda()
    combine_check(out, host(tr), gate, torch.bfloat16)
