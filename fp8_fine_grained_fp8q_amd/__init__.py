"""Python binding of libfp8q: online fine-grained E4M3 quantization and block-scaled FP8
GEMMs on AMD Instinct MI355X (gfx950).

The functions below carry the names of the C ABI (include/fp8q.h) and only marshal
arguments: PyTorch provides device memory and the current stream, every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the library is
missing or no GPU is present the calls raise.

    xq, sa = fp8q_quantize_act_1x128(x)            # x: bf16 [M, K] on cuda
    wq, sb = fp8q_quantize_w_128x128(w)            # w: bf16 [G, N, K] or [N, K]
    xq, sa, wq, sb = fp8q_quantize_act_w(x, w)     # both in one launch
    c = fp8q_gemm_blockscaled(xq, sa, wq, sb)      # bf16 [M, N] (or out_dtype=torch.float32)
    c = fp8q_grouped_gemm_blockscaled(xq, sa, wq, sb, offsets)   # offsets: int32 [G+1] on cuda

Backward pass (same E4M3 format):
    wq, sb, wqt, sbt = fp8q_quantize_w_128x128_t(w)   # also W^T codes / scales
    dx = fp8q_gemm_blockscaled(dyq, sa_dy, wqt, sbt)    # dgrad dX = dY W
    xq, sa, xqt, sat = fp8q_quantize_act_dual(x)        # tiles along K and along the tokens
    dw = fp8q_gemm_rowscaled(dyqt, sat_dy, xqt, sat)    # wgrad dW = dY^T X

Layouts: xq uint8 [M, K]; sa float32 [K/128, M]; wq uint8 [G, N, K]; sb float32
[G, N/128, K/128]; C row-major [M, N].
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# FP8Q_LIBRARY may point at another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("FP8Q_LIBRARY") or os.path.join(HERE, "libfp8q.so")

FP8Q_OK = 0
FP8Q_ERR_OFFSETS = -7  # grouped GEMM offsets rejected by the FP8Q_DEBUG check
FP8Q_OUT_BF16 = 0
FP8Q_OUT_F32 = 1
ABI_VERSION = 7

EXPORTED = ("fp8q_quantize_act_1x128", "fp8q_quantize_w_128x128", "fp8q_gemm_blockscaled",
            "fp8q_grouped_gemm_blockscaled", "fp8q_quantize_w_128x128_t", "fp8q_quantize_act_dual",
            "fp8q_gemm_rowscaled", "fp8q_swiglu_quantize_act_1x128", "fp8q_quantize_per_tensor",
            "fp8q_quantize_act_w", "fp8q_moe_dispatch", "fp8q_moe_combine", "fp8q_status_string",
            "fp8q_abi_version")


class Fp8qError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfp8q.so (built by fp8_fine_grained_fp8q_amd.build) and declare its C ABI."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libfp8q.so not found at {path}; build it with "
                           "`python -m fp8_fine_grained_fp8q_amd.build`")
    lib = ctypes.CDLL(path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32
    lib.fp8q_quantize_act_1x128.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.fp8q_quantize_w_128x128.argtypes = [vp, i64, i64, i64, vp, vp, vp]
    lib.fp8q_gemm_blockscaled.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i32, vp]
    lib.fp8q_grouped_gemm_blockscaled.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, vp]
    lib.fp8q_quantize_w_128x128_t.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.fp8q_quantize_act_dual.argtypes = [vp, i64, i64, vp, vp, vp, vp, vp]
    lib.fp8q_gemm_rowscaled.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, i32, vp]
    lib.fp8q_swiglu_quantize_act_1x128.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.fp8q_quantize_per_tensor.argtypes = [vp, i64, vp, vp, vp, vp]
    lib.fp8q_quantize_act_w.argtypes = [vp, i64, vp, i64, i64, i64, vp, vp, vp, vp, vp]
    lib.fp8q_moe_dispatch.argtypes = [vp, i64, i64, i64, i64, vp, vp, i64, i64, vp, vp, vp, vp, vp, vp]
    lib.fp8q_moe_combine.argtypes = [vp, i32, i64, i64, vp, vp, i64, i64, vp, i32, vp]
    for name in ("fp8q_quantize_act_1x128", "fp8q_quantize_w_128x128", "fp8q_gemm_blockscaled",
                 "fp8q_grouped_gemm_blockscaled", "fp8q_quantize_w_128x128_t", "fp8q_quantize_act_dual",
                 "fp8q_gemm_rowscaled", "fp8q_swiglu_quantize_act_1x128", "fp8q_quantize_per_tensor",
                 "fp8q_quantize_act_w", "fp8q_moe_dispatch", "fp8q_moe_combine"):
        getattr(lib, name).restype = i32
    lib.fp8q_status_string.argtypes = [i32]
    lib.fp8q_status_string.restype = ctypes.c_char_p
    lib.fp8q_abi_version.argtypes = []
    lib.fp8q_abi_version.restype = i32
    if lib.fp8q_abi_version() != ABI_VERSION:
        raise RuntimeError("libfp8q ABI version mismatch; rebuild the library")
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fp8q_status_string(int(status)).decode()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _check(status: int, what: str):
    if status != FP8Q_OK:
        raise Fp8qError(status, what)


def _need(t: torch.Tensor, dtype, name: str, shape=None):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def fp8q_quantize_act_1x128(x: torch.Tensor, xq: torch.Tensor | None = None,
                            sa: torch.Tensor | None = None, stream=None):
    """1x128 activation tiles -> (xq uint8 [M, K], sa float32 [K/128, M])."""
    _need(x, torch.bfloat16, "x")
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if sa is None:
        sa = torch.empty((K // 128, M), dtype=torch.float32, device=x.device)
    _need(xq, torch.uint8, "xq", (M, K))
    _need(sa, torch.float32, "sa", (K // 128, M))
    _check(load_library().fp8q_quantize_act_1x128(_ptr(x), M, K, _ptr(xq), _ptr(sa), _stream(stream)),
           "fp8q_quantize_act_1x128")
    return xq, sa


def fp8q_quantize_w_128x128(w: torch.Tensor, wq: torch.Tensor | None = None,
                            sb: torch.Tensor | None = None, stream=None):
    """128x128 weight blocks of w [G, N, K] (or [N, K]) -> (wq uint8, sb float32 [G, N/128, K/128])."""
    _need(w, torch.bfloat16, "w")
    squeeze = w.dim() == 2
    G, N, K = (1, *w.shape) if squeeze else w.shape
    if wq is None:
        wq = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    shape = (N // 128, K // 128) if squeeze else (G, N // 128, K // 128)
    if sb is None:
        sb = torch.empty(shape, dtype=torch.float32, device=w.device)
    _need(wq, torch.uint8, "wq", w.shape)
    _need(sb, torch.float32, "sb", shape)
    _check(load_library().fp8q_quantize_w_128x128(_ptr(w), G, N, K, _ptr(wq), _ptr(sb), _stream(stream)),
           "fp8q_quantize_w_128x128")
    return wq, sb


def fp8q_quantize_act_w(x: torch.Tensor, w: torch.Tensor, xq: torch.Tensor | None = None,
                        sa: torch.Tensor | None = None, wq: torch.Tensor | None = None,
                        sb: torch.Tensor | None = None, stream=None):
    """Both quantizers of a linear layer in one launch: x [M, K] -> (xq, sa) as
    fp8q_quantize_act_1x128 and w [G, N, K] (or [N, K]) -> (wq, sb) as fp8q_quantize_w_128x128."""
    _need(x, torch.bfloat16, "x")
    _need(w, torch.bfloat16, "w")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    squeeze = w.dim() == 2
    G, N, Kw = (1, *w.shape) if squeeze else w.shape
    if Kw != K:
        raise ValueError(f"x and w must share K, got {K} and {Kw}")
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if sa is None:
        sa = torch.empty((K // 128, M), dtype=torch.float32, device=x.device)
    if wq is None:
        wq = torch.empty(w.shape, dtype=torch.uint8, device=w.device)
    sb_shape = (N // 128, K // 128) if squeeze else (G, N // 128, K // 128)
    if sb is None:
        sb = torch.empty(sb_shape, dtype=torch.float32, device=w.device)
    _need(xq, torch.uint8, "xq", (M, K))
    _need(sa, torch.float32, "sa", (K // 128, M))
    _need(wq, torch.uint8, "wq", w.shape)
    _need(sb, torch.float32, "sb", sb_shape)
    _check(load_library().fp8q_quantize_act_w(_ptr(x), M, _ptr(w), G, N, K, _ptr(xq), _ptr(sa), _ptr(wq), _ptr(sb),
                                              _stream(stream)), "fp8q_quantize_act_w")
    return xq, sa, wq, sb


def fp8q_moe_dispatch(topk_ids: torch.Tensor, xq: torch.Tensor, sa: torch.Tensor, e_begin: int, n_experts: int,
                      capacity: int | None = None, stream=None):
    """Expert-parallel dispatch of quantized tokens to the local experts [e_begin,
    e_begin + n_experts): topk_ids int32 [T, k], xq uint8 [T, K], sa float32 [K/128, T] ->
    (xq_sorted uint8 [capacity, K], sa_sorted float32 [K/128, capacity], offsets int32
    [n_experts + 1], token_row int32 [T, k], row_token int32 [capacity]); capacity defaults
    to T*k.  offsets feed fp8q_grouped_gemm_blockscaled with the sorted tensors."""
    _need(topk_ids, torch.int32, "topk_ids")
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be 2-D [T, k]")
    T, k = topk_ids.shape
    _need(xq, torch.uint8, "xq")
    if xq.dim() != 2 or xq.shape[0] != T:
        raise ValueError(f"xq must be [T={T}, K]")
    K = xq.shape[1]
    _need(sa, torch.float32, "sa", (K // 128, T))
    cap = T * k if capacity is None else int(capacity)
    dev = xq.device
    xs = torch.empty((cap, K), dtype=torch.uint8, device=dev)
    ss = torch.empty((K // 128, cap), dtype=torch.float32, device=dev)
    offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    token_row = torch.empty((T, k), dtype=torch.int32, device=dev)
    row_token = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    _check(load_library().fp8q_moe_dispatch(_ptr(topk_ids), T, k, e_begin, n_experts, _ptr(xq), _ptr(sa), K, cap,
                                            _ptr(xs), _ptr(ss), _ptr(offsets), _ptr(token_row), _ptr(row_token),
                                            _stream(stream)), "fp8q_moe_dispatch")
    return xs, ss, offsets, token_row, row_token[:cap]


def fp8q_moe_combine(expert_out: torch.Tensor, token_row: torch.Tensor, topk_w: torch.Tensor,
                     y: torch.Tensor | None = None, out_dtype=torch.bfloat16, stream=None):
    """Expert-parallel combine: y[t] = sum over local slots of topk_w[t, s] * expert_out[token_row[t, s]]
    (expert_out bf16 or float32 [capacity, N]; token_row int32 / topk_w float32 [T, k])."""
    if expert_out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("expert_out must be bfloat16 or float32")
    _need(expert_out, expert_out.dtype, "expert_out")
    _need(token_row, torch.int32, "token_row")
    if token_row.dim() != 2 or expert_out.dim() != 2:
        raise ValueError("token_row must be [T, k] and expert_out [capacity, N]")
    T, k = token_row.shape
    cap, N = expert_out.shape
    _need(topk_w, torch.float32, "topk_w", (T, k))
    if y is None:
        y = torch.empty((T, N), dtype=out_dtype, device=expert_out.device)
    _need(y, out_dtype, "y", (T, N))
    _check(load_library().fp8q_moe_combine(_ptr(expert_out), _out_code(expert_out.dtype), cap, N, _ptr(token_row),
                                           _ptr(topk_w), T, k, _ptr(y), _out_code(out_dtype), _stream(stream)),
           "fp8q_moe_combine")
    return y


def _out_code(out_dtype) -> int:
    if out_dtype == torch.bfloat16:
        return FP8Q_OUT_BF16
    if out_dtype == torch.float32:
        return FP8Q_OUT_F32
    raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")


def fp8q_gemm_blockscaled(xq, sa, wq, sb, out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
                          stream=None):
    """C = dequant(xq, sa) @ dequant(wq, sb)^T with FP32 promotion per 128-wide K block."""
    _need(xq, torch.uint8, "xq")
    _need(wq, torch.uint8, "wq")
    _need(sa, torch.float32, "sa")
    _need(sb, torch.float32, "sb")
    M, K = xq.shape
    if wq.dim() == 3 and wq.shape[0] == 1:
        wq, sb = wq[0], sb.reshape(sb.shape[-2:])
    if wq.dim() != 2:
        raise ValueError("the dense GEMM takes one weight matrix wq [N, K]; use the grouped GEMM for experts")
    N = wq.shape[0]
    _need(wq, torch.uint8, "wq", (N, K))
    _need(sa, torch.float32, "sa", (K // 128, M))
    _need(sb, torch.float32, "sb", (N // 128, K // 128))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    _need(out, out.dtype, "out", (M, N))
    _check(load_library().fp8q_gemm_blockscaled(_ptr(xq), _ptr(sa), _ptr(wq), _ptr(sb), M, N, K, _ptr(out),
                                                _out_code(out.dtype), _stream(stream)),
           "fp8q_gemm_blockscaled")
    return out


def fp8q_grouped_gemm_blockscaled(xq, sa, wq, sb, offsets, out_dtype=torch.bfloat16,
                                  out: torch.Tensor | None = None, stream=None):
    """Grouped (MoE): rows offsets[g]..offsets[g+1]-1 use expert g's weights wq[g], sb[g]."""
    _need(xq, torch.uint8, "xq")
    _need(wq, torch.uint8, "wq")
    _need(sa, torch.float32, "sa")
    _need(sb, torch.float32, "sb")
    _need(offsets, torch.int32, "offsets")
    M, K = xq.shape
    G, N, _ = wq.shape
    _need(wq, torch.uint8, "wq", (G, N, K))
    _need(sa, torch.float32, "sa", (K // 128, M))
    _need(sb, torch.float32, "sb", (G, N // 128, K // 128))
    _need(offsets, torch.int32, "offsets", (G + 1,))
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    _need(out, out.dtype, "out", (M, N))
    _check(load_library().fp8q_grouped_gemm_blockscaled(
        _ptr(xq), _ptr(sa), _ptr(wq), _ptr(sb), _ptr(offsets), G, M, N, K, _ptr(out),
        _out_code(out.dtype), _stream(stream)), "fp8q_grouped_gemm_blockscaled")
    return out


def fp8q_quantize_w_128x128_t(w: torch.Tensor, wq=None, sb=None, wqt=None, sbt=None, stream=None):
    """128x128 blocks of w [G, N, K] (or [N, K]) -> (wq, sb, wqt, sbt): the codes and scales
    of w and of its transpose (wqt uint8 [G, K, N], sbt float32 [G, K/128, N/128])."""
    _need(w, torch.bfloat16, "w")
    squeeze = w.dim() == 2
    G, N, K = (1, *w.shape) if squeeze else w.shape
    lead = () if squeeze else (G,)
    dev = w.device
    wq = torch.empty(w.shape, dtype=torch.uint8, device=dev) if wq is None else wq
    sb = torch.empty(lead + (N // 128, K // 128), dtype=torch.float32, device=dev) if sb is None else sb
    wqt = torch.empty(lead + (K, N), dtype=torch.uint8, device=dev) if wqt is None else wqt
    sbt = torch.empty(lead + (K // 128, N // 128), dtype=torch.float32, device=dev) if sbt is None else sbt
    _need(wq, torch.uint8, "wq", w.shape)
    _need(sb, torch.float32, "sb", lead + (N // 128, K // 128))
    _need(wqt, torch.uint8, "wqt", lead + (K, N))
    _need(sbt, torch.float32, "sbt", lead + (K // 128, N // 128))
    _check(load_library().fp8q_quantize_w_128x128_t(_ptr(w), G, N, K, _ptr(wq), _ptr(sb), _ptr(wqt), _ptr(sbt),
                                                    _stream(stream)), "fp8q_quantize_w_128x128_t")
    return wq, sb, wqt, sbt


def fp8q_quantize_act_dual(x: torch.Tensor, xq=None, sa=None, xqt=None, sat=None, stream=None):
    """x bf16 [M, K] (M % 128 == 0) -> (xq [M, K], sa [K/128, M], xqt [K, M], sat [M/128, K]):
    1x128 tiles along K and tiles of 128 tokens along M (codes channel-major)."""
    _need(x, torch.bfloat16, "x")
    M, K = x.shape
    dev = x.device
    xq = torch.empty((M, K), dtype=torch.uint8, device=dev) if xq is None else xq
    sa = torch.empty((K // 128, M), dtype=torch.float32, device=dev) if sa is None else sa
    xqt = torch.empty((K, M), dtype=torch.uint8, device=dev) if xqt is None else xqt
    sat = torch.empty((M // 128, K), dtype=torch.float32, device=dev) if sat is None else sat
    _need(xq, torch.uint8, "xq", (M, K))
    _need(sa, torch.float32, "sa", (K // 128, M))
    _need(xqt, torch.uint8, "xqt", (K, M))
    _need(sat, torch.float32, "sat", (M // 128, K))
    _check(load_library().fp8q_quantize_act_dual(_ptr(x), M, K, _ptr(xq), _ptr(sa), _ptr(xqt), _ptr(sat),
                                                 _stream(stream)), "fp8q_quantize_act_dual")
    return xq, sa, xqt, sat


def fp8q_gemm_rowscaled(aq, sa, bq, sb, out_dtype=torch.bfloat16, out: torch.Tensor | None = None, stream=None):
    """C [P, Q] = dequant(aq, sa) @ dequant(bq, sb)^T with 1x128 row scales on both operands:
    aq [P, Kc], sa [Kc/128, P], bq [Q, Kc], sb [Kc/128, Q]."""
    _need(aq, torch.uint8, "aq")
    _need(bq, torch.uint8, "bq")
    _need(sa, torch.float32, "sa")
    _need(sb, torch.float32, "sb")
    P, Kc = aq.shape
    Q = bq.shape[0]
    _need(bq, torch.uint8, "bq", (Q, Kc))
    _need(sa, torch.float32, "sa", (Kc // 128, P))
    _need(sb, torch.float32, "sb", (Kc // 128, Q))
    if out is None:
        out = torch.empty((P, Q), dtype=out_dtype, device=aq.device)
    _need(out, out.dtype, "out", (P, Q))
    _check(load_library().fp8q_gemm_rowscaled(_ptr(aq), _ptr(sa), _ptr(bq), _ptr(sb), P, Q, Kc, _ptr(out),
                                              _out_code(out.dtype), _stream(stream)), "fp8q_gemm_rowscaled")
    return out


def fp8q_swiglu_quantize_act_1x128(gu: torch.Tensor, xq=None, sa=None, stream=None):
    """gu bf16 [M, 2I] (g | u) -> (xq uint8 [M, I], sa float32 [I/128, M]) for h = SiLU(g) * u."""
    _need(gu, torch.bfloat16, "gu")
    M, I2 = gu.shape
    I = I2 // 2
    xq = torch.empty((M, I), dtype=torch.uint8, device=gu.device) if xq is None else xq
    sa = torch.empty((I // 128, M), dtype=torch.float32, device=gu.device) if sa is None else sa
    _need(xq, torch.uint8, "xq", (M, I))
    _need(sa, torch.float32, "sa", (I // 128, M))
    _check(load_library().fp8q_swiglu_quantize_act_1x128(_ptr(gu), M, I, _ptr(xq), _ptr(sa), _stream(stream)),
           "fp8q_swiglu_quantize_act_1x128")
    return xq, sa


def fp8q_quantize_per_tensor(x: torch.Tensor, scale: torch.Tensor | None = None, q=None, stats=None, stream=None):
    """One scale for all of x (bf16, any shape, numel % 8 == 0): tensor-level scaling when
    `scale` is None, else delayed scaling with that device float32 scale.  Returns
    (q uint8 like x, stats int32 [3]: amax bits, saturated count, scale bits)."""
    _need(x, torch.bfloat16, "x")
    if scale is not None:
        _need(scale, torch.float32, "scale")
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if q is None else q
    stats = torch.empty(3, dtype=torch.int32, device=x.device) if stats is None else stats
    _need(q, torch.uint8, "q", x.shape)
    _need(stats, torch.int32, "stats", (3,))
    if scale is not None and scale.numel() != 1:
        raise ValueError("scale must hold one float32")
    _check(load_library().fp8q_quantize_per_tensor(_ptr(x), x.numel(), _ptr(scale), _ptr(q), _ptr(stats),
                                                   _stream(stream)), "fp8q_quantize_per_tensor")
    return q, stats


def tensor_stats(stats: torch.Tensor):
    """(amax, saturated count, scale) of a stats tensor from fp8q_quantize_per_tensor."""
    h = stats.cpu()
    return (float(h[0:1].view(torch.float32)), int(h[1]), float(h[2:3].view(torch.float32)))


quantize_act_1x128 = fp8q_quantize_act_1x128
quantize_w_128x128 = fp8q_quantize_w_128x128
gemm_blockscaled = fp8q_gemm_blockscaled
grouped_gemm_blockscaled = fp8q_grouped_gemm_blockscaled
quantize_w_128x128_t = fp8q_quantize_w_128x128_t
quantize_act_dual = fp8q_quantize_act_dual
gemm_rowscaled = fp8q_gemm_rowscaled
swiglu_quantize_act_1x128 = fp8q_swiglu_quantize_act_1x128
quantize_per_tensor = fp8q_quantize_per_tensor
