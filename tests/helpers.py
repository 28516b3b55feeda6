"""Helpers shared by the GPU tests: moving seeded numpy inputs to the device and comparing
GPU results with the oracle."""
import numpy as np
import torch

from oracle import gemm as ogemm


def dev_bf16(u16: np.ndarray) -> torch.Tensor:
    """uint16 BF16 patterns (numpy) -> contiguous bf16 CUDA tensor with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().numpy().astype(np.float64)
    return t.numpy()


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_quant_equal(xq_gpu, s_gpu, xq_ref, s_ref, what=""):
    """Bit-exact comparison of codes and scales (scales compared as bit patterns)."""
    q = host(xq_gpu)
    s = host(s_gpu)
    assert q.shape == xq_ref.shape and s.shape == s_ref.shape, what
    bad_s = np.nonzero(f32_bits(s) != f32_bits(s_ref))
    assert bad_s[0].size == 0, f"{what}: {bad_s[0].size} scales differ, first at {[b[0] for b in bad_s]}: gpu {s[tuple(b[0] for b in bad_s)]!r} ref {s_ref[tuple(b[0] for b in bad_s)]!r}"
    bad = np.nonzero(q != xq_ref)
    assert bad[0].size == 0, f"{what}: {bad[0].size} codes differ, first at {[int(b[0]) for b in bad]}: gpu {hex(q[tuple(b[0] for b in bad)])} ref {hex(xq_ref[tuple(b[0] for b in bad)])}"


def assert_gemm_within_tol(c_gpu: np.ndarray, c_ref: np.ndarray, xnorm, wnorm, what=""):
    """|C_gpu - C_ref| <= 2e-3 * ||x_hat_m|| * ||w_hat_n|| element-wise (C_gpu as stored)."""
    tol = ogemm.tolerance(xnorm, wnorm)
    assert c_gpu.shape == c_ref.shape == tol.shape, what
    assert np.all(np.isfinite(c_gpu)), what
    err = np.abs(c_gpu - c_ref)
    worst = np.unravel_index(np.argmax(err / np.maximum(tol, 1e-300)), err.shape)
    assert np.all(err <= tol), (f"{what}: {np.count_nonzero(err > tol)} elements out of tolerance; "
                                f"worst at {worst}: gpu {c_gpu[worst]} ref {c_ref[worst]} tol {tol[worst]}")
    ratio = float(np.max(err / np.maximum(tol, 1e-300)))
    print(f"[{what}] max |err|/tol = {ratio:.4f}", flush=True)
    return ratio
