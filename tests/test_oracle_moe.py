"""Pins for the oracle's expert-parallel dispatch and combine (CPU only): brute-force loops,
the per-expert token lists the workloads derive from the same routing, row-locality of the
activation quantizer (quantize-then-pack equals pack-then-quantize), and closed forms of
the combine."""
import numpy as np

import workloads as wl
from oracle import moe as om
from oracle import quant as oq


def brute_dispatch(ids, e_begin, E):
    T, k = ids.shape
    rows = []
    for e in range(E):
        for t in range(T):
            for s in range(k):
                if ids[t, s] == e_begin + e:
                    rows.append((e, t, s))
    return rows


def test_dispatch_matches_brute_force():
    rng = np.random.default_rng(3)
    T, k, E, e_begin = 37, 4, 6, 5
    ids = np.stack([rng.choice(16, k, replace=False) for _ in range(T)]).astype(np.int32)
    offsets, row_token, token_row = om.dispatch(ids, e_begin, E)
    rows = brute_dispatch(ids, e_begin, E)
    assert offsets[-1] == len(rows)
    for r, (e, t, s) in enumerate(rows):
        assert offsets[e] <= r < offsets[e + 1]
        assert row_token[r] == t and token_row[t, s] == r
    local = (ids >= e_begin) & (ids < e_begin + E)
    assert np.all(token_row[~local] == -1)


def test_dispatch_agrees_with_workload_routing_lists():
    """The moe_up workload lists, per local expert, the tokens routed to it; the dispatch of
    the same top-8 ids must give the same rows in the same order."""
    ids, _ = wl.topk_routing(tokens=512)
    rows, offsets_ref = wl.routing(tokens=512, local=32)
    offsets, row_token, _ = om.dispatch(ids, 0, 32)
    assert np.array_equal(offsets, offsets_ref)
    assert np.array_equal(row_token, np.concatenate(rows))


def test_dispatch_without_local_experts():
    ids = np.array([[40, 41], [42, 43]], np.int32)
    offsets, row_token, token_row = om.dispatch(ids, 0, 32)
    assert np.all(offsets == 0) and row_token.size == 0 and np.all(token_row == -1)


def test_pack_commutes_with_the_row_local_quantizer():
    rng = np.random.default_rng(4)
    T, K = 20, 384
    x = wl.bf16_bits(rng.standard_normal((T, K), dtype=np.float32) * np.float32(5.0))
    ids = np.stack([rng.choice(12, 3, replace=False) for _ in range(T)]).astype(np.int32)
    _, row_token, _ = om.dispatch(ids, 2, 8)
    xq, sa = oq.quantize_act_1x128(x)
    pq, psa = om.pack(xq, sa, row_token)
    rq, rsa = oq.quantize_act_1x128(x[row_token])
    assert np.array_equal(pq, rq) and np.array_equal(psa.view(np.uint32), rsa.view(np.uint32))


def test_combine_closed_forms():
    # one slot per token, all local: y = w * out[row]
    out = np.arange(12, dtype=np.float64).reshape(4, 3) + 1.0
    token_row = np.array([[2], [0], [3], [1]], np.int32)
    w = np.array([[0.5], [2.0], [-1.0], [0.25]], np.float32)
    y = om.combine(out, token_row, w)
    assert np.array_equal(y, w.astype(np.float64) * out[token_row[:, 0]])
    # constant outputs, unit weights: y = (number of local slots) * c; non-local slots add nothing
    out = np.full((5, 4), 3.0)
    token_row = np.array([[0, 1, -1], [2, -1, -1], [-1, -1, -1], [3, 4, 0]], np.int32)
    y = om.combine(out, token_row, np.ones((4, 3), np.float32))
    assert np.array_equal(y[:, 0], np.array([6.0, 3.0, 0.0, 9.0]))


def test_combine_matches_loop():
    rng = np.random.default_rng(5)
    T, k, R, N = 9, 4, 20, 6
    out = rng.standard_normal((R, N))
    token_row = rng.integers(-1, R, size=(T, k)).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    y = om.combine(out, token_row, w)
    for t in range(T):
        ref = np.zeros(N)
        for s in range(k):
            if token_row[t, s] >= 0:
                ref += float(w[t, s]) * out[token_row[t, s]]
        assert np.allclose(y[t], ref, rtol=0, atol=1e-12)
    assert np.all(om.combine_bound(out, token_row, w) >= np.abs(y) - 1e-12)
