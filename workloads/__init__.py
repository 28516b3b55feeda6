"""Seeded synthetic inputs for the fine-grained FP8 quantization + block-scaled GEMM path.

This module only *draws* inputs.  It holds none of the method's arithmetic
(no scaling, no FP8 coding, no products), so both the CPU oracle and the GPU
path can take their inputs from here without sharing any of the computation.

Every tensor is drawn in FP32 with numpy's PCG64 (``default_rng``), one child
``SeedSequence`` per tensor, then rounded to BF16 (round to nearest, ties to
even) and returned as the raw 16-bit patterns (``uint16``).  The shapes and
value distributions are those of the five workloads the path is measured on:

    tiny      X[128x512]  N(0,1), 1% of entries x50;  W[256x512]  N(0,0.02); BF16 out
    dense     X[4096x7168] N(0,1), 8 fixed channels x100;  W[7168x7168] N(0,0.02); BF16 out
    moe_up    8192 tokens x 7168, N(0,1) logits -> softmax + per-expert bias -> top-8 of 256,
              the 32 local experts kept; W[32][4096x7168] N(0,0.02); BF16 out
    moe_down  same routing; input SiLU(g)*u [n x 2048]; W[32][7168x2048] N(0,0.02); BF16 out
    large     X[16384x7168] Student-t(3);  W[18432x7168] N(0,0.02); FP32 out

The DeepSeek-V3 pages describe the model these stand in for (MoE layers with
256 routed experts of which 8 are active per token, hidden size not given) but
publish no data; nothing here is taken from a dataset.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

SEEDS = {"tiny": 1, "dense": 2, "moe_up": 3, "moe_down": 4, "large": 5, "train": 6}


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round an FP32 array to BF16 (nearest, ties to even) and return the 16-bit patterns.

    Inputs are finite by construction; no NaN handling is needed here."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _rngs(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return bf16_bits(a)


def _weights(seed_rng_list, G: int, N: int, K: int, std: float = 0.02) -> np.ndarray:
    """G independent N(0,std) weight matrices, one child generator each (thread-parallel,
    deterministic whatever the thread count)."""
    out = np.empty((G, N, K), dtype=np.uint16)

    def one(g):
        out[g] = normal_bf16(seed_rng_list[g], (N, K), std)

    with _cf.ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(one, range(G)))
    return out


def tiny(seed: int = SEEDS["tiny"]):
    r_x, r_mask, r_w = _rngs(seed, 3)
    x = r_x.standard_normal((128, 512), dtype=np.float32)
    mask = r_mask.random((128, 512)) < 0.01
    x[mask] *= np.float32(50.0)
    w = r_w.standard_normal((256, 512), dtype=np.float32) * np.float32(0.02)
    return {"name": "tiny", "x": bf16_bits(x), "w": bf16_bits(w)[None], "offsets": None,
            "out_dtype": "bf16"}


def dense(seed: int = SEEDS["dense"], M: int = 4096, N: int = 7168, K: int = 7168):
    r_x, r_ch, r_w = _rngs(seed, 3)
    x = r_x.standard_normal((M, K), dtype=np.float32)
    # 8 fixed outlier channels (whole columns) scaled x100: 8/7168 ~ 0.1% of entries
    ch = r_ch.choice(K, size=8, replace=False)
    x[:, ch] *= np.float32(100.0)
    w = _weights(_rngs(seed * 1000 + 7, 1), 1, N, K)
    return {"name": "dense", "x": bf16_bits(x), "w": w, "offsets": None, "out_dtype": "bf16",
            "outlier_channels": np.sort(ch)}


def topk_routing(seed: int = SEEDS["moe_up"], tokens: int = 8192, experts: int = 256, topk: int = 8,
                 bias_std: float = 0.003):
    """Top-8-of-256 routing from N(0,1) logits: softmax scores plus a static per-expert bias
    (used for selection only), ties to the lower expert index.  Returns the selected expert
    ids [tokens][topk] (int32, by decreasing biased score) and their gating weights (the
    unbiased scores of the selected experts normalised to sum to 1 per token, float32)."""
    r_logit, r_bias = _rngs(seed + 100, 2)
    logits = r_logit.standard_normal((tokens, experts))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    score = e / e.sum(axis=1, keepdims=True)
    bias = bias_std * r_bias.standard_normal(experts)
    sel = np.argsort(-(score + bias), axis=1, kind="stable")[:, :topk]
    g = np.take_along_axis(score, sel, axis=1)
    return sel.astype(np.int32), (g / g.sum(axis=1, keepdims=True)).astype(np.float32)


def routing(seed: int = SEEDS["moe_up"], tokens: int = 8192, experts: int = 256, topk: int = 8,
            local: int = 32, bias_std: float = 0.003):
    """For the first ``local`` experts of topk_routing: the token ids routed to each
    (ascending) and the offsets array."""
    sel, _ = topk_routing(seed, tokens, experts, topk, bias_std)
    rows = []
    for g in range(local):
        rows.append(np.nonzero((sel == g).any(axis=1))[0].astype(np.int64))
    counts = np.array([len(r) for r in rows], dtype=np.int64)
    offsets = np.zeros(local + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return rows, offsets


def moe_up(seed: int = SEEDS["moe_up"], tokens: int = 8192, hidden: int = 7168, N: int = 4096,
           local: int = 32):
    rows, offsets = routing(seed, tokens=tokens, local=local)
    r_x, = _rngs(seed, 1)
    tok = r_x.standard_normal((tokens, hidden), dtype=np.float32)
    order = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    x = bf16_bits(tok[order])
    w = _weights(_rngs(seed * 1000 + 7, local), local, N, hidden)
    return {"name": "moe_up", "x": x, "w": w, "offsets": offsets, "out_dtype": "bf16"}


def moe_down(seed: int = SEEDS["moe_down"], route_seed: int = SEEDS["moe_up"], tokens: int = 8192,
             inter: int = 2048, N: int = 7168, local: int = 32):
    rows, offsets = routing(route_seed, tokens=tokens, local=local)
    m = int(offsets[-1])
    r_g, r_u = _rngs(seed, 2)
    g = r_g.standard_normal((m, inter), dtype=np.float32)
    u = r_u.standard_normal((m, inter), dtype=np.float32)
    act = (g / (np.float32(1.0) + np.exp(-g))) * u  # SiLU(g) * u
    w = _weights(_rngs(seed * 1000 + 7, local), local, N, inter)
    return {"name": "moe_down", "x": bf16_bits(act), "w": w, "offsets": offsets,
            "out_dtype": "bf16"}


def large(seed: int = SEEDS["large"], M: int = 16384, N: int = 18432, K: int = 7168):
    r_x, r_w = _rngs(seed, 2)
    x = r_x.standard_t(3.0, size=(M, K)).astype(np.float32)
    w = _weights(_rngs(seed * 1000 + 7, 1), 1, N, K)
    return {"name": "large", "x": bf16_bits(x), "w": w, "offsets": None, "out_dtype": "f32"}


def moe_layer(seed: int = SEEDS["moe_up"], tokens: int = 8192, hidden: int = 7168, inter: int = 2048,
              local: int = 32):
    """One GPU's share of the MoE expert layer from the token side: the moe_up tokens in
    token order X[tokens][hidden], their top-8 routing (global expert ids and gating
    weights), and the 32 local experts' W_up[32][2*inter x hidden] and W_down[32][hidden x inter]."""
    ids, gate = topk_routing(seed, tokens=tokens)
    r_x, = _rngs(seed, 1)
    x = bf16_bits(r_x.standard_normal((tokens, hidden), dtype=np.float32))
    w_up = _weights(_rngs(seed * 1000 + 7, local), local, 2 * inter, hidden)
    w_down = _weights(_rngs(SEEDS["moe_down"] * 1000 + 7, local), local, hidden, inter)
    return {"name": "moe_layer", "x": x, "topk_ids": ids, "topk_w": gate, "e_begin": 0, "local": local,
            "w": w_up, "w_down": w_down, "offsets": None, "out_dtype": "bf16"}


def moe_ffn(seed: int = SEEDS["moe_up"]):
    """The expert FFN forward of the 32 local experts: the moe_up input and up-projection
    weights plus the moe_down workload's down-projection weights W_down[32][7168x2048]."""
    up = moe_up(seed)
    G, N1, K = up["w"].shape
    w_down = _weights(_rngs(SEEDS["moe_down"] * 1000 + 7, G), G, K, N1 // 2)
    return {"name": "moe_ffn", "x": up["x"], "w": up["w"], "w_down": w_down, "offsets": up["offsets"],
            "out_dtype": "bf16"}


def train(seed: int = SEEDS["train"], M: int = 4096, N: int = 7168, K: int = 7168):
    """One training step of the dense projection: the dense workload's X and W plus an
    output gradient dY[M][N] (N(0,1) x 1e-3, with the rows of 16 tokens scaled x50 so the
    token tiles see outliers too)."""
    c = dense(M=M, N=N, K=K)
    r_dy, r_tok = _rngs(seed, 2)
    dy = r_dy.standard_normal((M, N), dtype=np.float32) * np.float32(1e-3)
    tok = r_tok.choice(M, size=16, replace=False)
    dy[tok] *= np.float32(50.0)
    c.update({"name": "train", "dy": bf16_bits(dy), "out_dtype": "bf16"})
    return c


CONFIGS = {"tiny": tiny, "dense": dense, "moe_up": moe_up, "moe_down": moe_down, "large": large, "train": train,
           "moe_ffn": moe_ffn, "moe_layer": moe_layer}
