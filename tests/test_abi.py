"""C ABI checks that need no GPU: the library loads, exports every function the header
declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

import fp8_fine_grained_fp8q_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")

ALIGNED = 1 << 20  # a fake, 16-byte aligned device address (never dereferenced)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8q_[a-z0-9_]+)\s*\(", text)))


def header_enums():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"\b(FP8Q_[A-Z0-9_]+)\s*=\s*(-?\d+)", text)}


@pytest.fixture(scope="module")
def lib():
    return fq.load_library()


def test_library_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == set(fq.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fq.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fp8q_[a-z0-9_]+)\b", out))
    assert set(names) <= exported


def test_enum_values_match_binding(lib):
    e = header_enums()
    assert e["FP8Q_OK"] == fq.FP8Q_OK == 0
    assert e["FP8Q_OUT_BF16"] == fq.FP8Q_OUT_BF16 and e["FP8Q_OUT_F32"] == fq.FP8Q_OUT_F32
    assert lib.fp8q_abi_version() == fq.ABI_VERSION
    assert e["FP8Q_ERR_OFFSETS"] == fq.FP8Q_ERR_OFFSETS
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -99):
        assert isinstance(fq.status_string(code), str) and fq.status_string(code)
    assert "offsets" in fq.status_string(fq.FP8Q_ERR_OFFSETS)


def test_quantize_act_argument_checks(lib):
    E = header_enums()
    A = ALIGNED
    assert lib.fp8q_quantize_act_1x128(A, 4, 100, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert lib.fp8q_quantize_act_1x128(A, -1, 128, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert lib.fp8q_quantize_act_1x128(A, 1 << 40, 1 << 30, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert lib.fp8q_quantize_act_1x128(None, 4, 128, A, A, None) == E["FP8Q_ERR_NULL"]
    assert lib.fp8q_quantize_act_1x128(A, 4, 128, None, A, None) == E["FP8Q_ERR_NULL"]
    assert lib.fp8q_quantize_act_1x128(A + 2, 4, 128, A, A, None) == E["FP8Q_ERR_ALIGN"]
    assert lib.fp8q_quantize_act_1x128(A, 4, 128, A, A + 4, None) == E["FP8Q_ERR_ALIGN"]
    # empty work is a no-op, even with null buffers
    assert lib.fp8q_quantize_act_1x128(None, 0, 128, None, None, None) == E["FP8Q_OK"]
    assert lib.fp8q_quantize_act_1x128(None, 5, 0, None, None, None) == E["FP8Q_OK"]


def test_quantize_w_argument_checks(lib):
    E = header_enums()
    A = ALIGNED
    assert lib.fp8q_quantize_w_128x128(A, 0, 128, 128, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert lib.fp8q_quantize_w_128x128(A, 1, 100, 128, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert lib.fp8q_quantize_w_128x128(A, 1, 128, 64, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert lib.fp8q_quantize_w_128x128(None, 1, 128, 128, A, A, None) == E["FP8Q_ERR_NULL"]
    assert lib.fp8q_quantize_w_128x128(A, 1, 128, 128, A, A + 8, None) == E["FP8Q_ERR_ALIGN"]
    assert lib.fp8q_quantize_w_128x128(None, 3, 0, 128, None, None, None) == E["FP8Q_OK"]


def test_gemm_argument_checks(lib):
    E = header_enums()
    A = ALIGNED
    g = lib.fp8q_gemm_blockscaled
    assert g(A, A, A, A, 4, 128, 128, A, 7, None) == E["FP8Q_ERR_DTYPE"]
    assert g(A, A, A, A, 4, 100, 128, A, 0, None) == E["FP8Q_ERR_SHAPE"]
    assert g(A, A, A, A, 4, 128, 0, A, 0, None) == E["FP8Q_ERR_SHAPE"]
    assert g(A, A, A, A, 4, 128, 200, A, 0, None) == E["FP8Q_ERR_SHAPE"]
    assert g(A, A, A, A, -4, 128, 128, A, 0, None) == E["FP8Q_ERR_SHAPE"]
    assert g(A, A, None, A, 4, 128, 128, A, 0, None) == E["FP8Q_ERR_NULL"]
    assert g(A, A, A, A, 4, 128, 128, None, 0, None) == E["FP8Q_ERR_NULL"]
    assert g(A, A, A + 1, A, 4, 128, 128, A, 0, None) == E["FP8Q_ERR_ALIGN"]
    assert g(None, None, None, None, 0, 128, 128, None, 0, None) == E["FP8Q_OK"]
    assert g(A, A, A, A, 4, 128, (1 << 22) + 128, A, 0, None) == E["FP8Q_ERR_SHAPE"]   # 32-bit stage offsets
    assert lib.fp8q_gemm_rowscaled(A, A, A, A, 4, 128, (1 << 22) + 128, A, 0, None) == E["FP8Q_ERR_SHAPE"]
    gg = lib.fp8q_grouped_gemm_blockscaled
    assert gg(A, A, A, A, A, 0, 4, 128, 128, A, 0, None) == E["FP8Q_ERR_SHAPE"]
    assert gg(A, A, A, A, None, 2, 4, 128, 128, A, 0, None) == E["FP8Q_ERR_NULL"]
    assert gg(A, A, A, A, A + 2, 2, 4, 128, 128, A, 1, None) == E["FP8Q_ERR_ALIGN"]
    assert gg(A, A, A, A, A, 2, 4, 128, 128, A, 3, None) == E["FP8Q_ERR_DTYPE"]
    assert gg(None, None, None, None, None, 2, 0, 128, 128, None, 0, None) == E["FP8Q_OK"]


def test_backward_entry_point_argument_checks(lib):
    E = header_enums()
    A = ALIGNED
    t = lib.fp8q_quantize_w_128x128_t
    assert t(A, 1, 100, 128, A, A, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert t(A, 0, 128, 128, A, A, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert t(A, 1, 128, 128, A, A, None, A, None) == E["FP8Q_ERR_NULL"]
    assert t(A, 1, 128, 128, A, A, A, None, None) == E["FP8Q_ERR_NULL"]
    assert t(A, 1, 128, 128, A, A, A + 4, A, None) == E["FP8Q_ERR_ALIGN"]
    assert t(None, 1, 0, 128, None, None, None, None, None) == E["FP8Q_OK"]
    d = lib.fp8q_quantize_act_dual
    assert d(A, 200, 128, A, A, A, A, None) == E["FP8Q_ERR_SHAPE"]   # tokens not a multiple of 128
    assert d(A, 256, 100, A, A, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert d(A, 256, 128, A, A, None, A, None) == E["FP8Q_ERR_NULL"]
    assert d(A, 256, 128, A, A, A, A + 8, None) == E["FP8Q_ERR_ALIGN"]
    assert d(None, 0, 128, None, None, None, None, None) == E["FP8Q_OK"]
    r = lib.fp8q_gemm_rowscaled
    assert r(A, A, A, A, 4, 128, 128, A, 5, None) == E["FP8Q_ERR_DTYPE"]
    assert r(A, A, A, A, 4, 100, 128, A, 0, None) == E["FP8Q_ERR_SHAPE"]
    assert r(A, A, A, A, 4, 128, 64, A, 0, None) == E["FP8Q_ERR_SHAPE"]
    assert r(A, A, A, A, 4, 1 << 20, 1 << 17, A, 0, None) == E["FP8Q_ERR_SHAPE"]  # scale offsets too large
    assert r(A, None, A, A, 4, 128, 128, A, 0, None) == E["FP8Q_ERR_NULL"]
    assert r(A, A, A, A + 4, 4, 128, 128, A, 0, None) == E["FP8Q_ERR_ALIGN"]
    assert r(None, None, None, None, 0, 128, 128, None, 0, None) == E["FP8Q_OK"]


def test_swiglu_quantizer_argument_checks(lib):
    E = header_enums()
    A = ALIGNED
    f = lib.fp8q_swiglu_quantize_act_1x128
    assert f(A, 4, 100, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert f(A, -1, 128, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert f(None, 4, 128, A, A, None) == E["FP8Q_ERR_NULL"]
    assert f(A, 4, 128, A, None, None) == E["FP8Q_ERR_NULL"]
    assert f(A + 2, 4, 128, A, A, None) == E["FP8Q_ERR_ALIGN"]
    assert f(None, 0, 128, None, None, None) == E["FP8Q_OK"]


def test_per_tensor_quantizer_argument_checks(lib):
    E = header_enums()
    A = ALIGNED
    f = lib.fp8q_quantize_per_tensor
    assert f(A, 12, None, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert f(A, -8, None, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert f(A, 64, None, A, None, None) == E["FP8Q_ERR_NULL"]
    assert f(None, 64, None, A, A, None) == E["FP8Q_ERR_NULL"]
    assert f(A + 8, 64, None, A, A, None) == E["FP8Q_ERR_ALIGN"]
    assert f(A, 64, A + 2, A, A, None) == E["FP8Q_ERR_ALIGN"]


def test_fused_quantizer_argument_checks(lib):
    r = lib.fp8q_quantize_act_w
    A = ALIGNED
    E = header_enums()
    assert r(A, 4, A, 1, 128, 100, A, A, A, A, None) == E["FP8Q_ERR_SHAPE"]    # K % 128
    assert r(A, 4, A, 1, 100, 128, A, A, A, A, None) == E["FP8Q_ERR_SHAPE"]    # N % 128
    assert r(A, 4, A, 0, 128, 128, A, A, A, A, None) == E["FP8Q_ERR_SHAPE"]    # G < 1
    assert r(A, -1, A, 1, 128, 128, A, A, A, A, None) == E["FP8Q_ERR_SHAPE"]
    assert r(0, 0, A, 1, 0, 128, 0, 0, 0, 0, None) == E["FP8Q_OK"]            # nothing to do
    assert r(0, 4, A, 1, 128, 128, A, A, A, A, None) == E["FP8Q_ERR_NULL"]     # x
    assert r(A, 4, 0, 1, 128, 128, A, A, A, A, None) == E["FP8Q_ERR_NULL"]     # w
    assert r(A, 4, A, 1, 128, 128, A, A, A, 0, None) == E["FP8Q_ERR_NULL"]     # sb
    assert r(A + 4, 4, A, 1, 128, 128, A, A, A, A, None) == E["FP8Q_ERR_ALIGN"]
    assert r(A, 4, A, 1, 128, 128, A, A, A + 8, A, None) == E["FP8Q_ERR_ALIGN"]


def test_valid_call_without_gpu_reports_device_error(lib):
    """On a host without a GPU a well-formed call must fail cleanly, not crash."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    E = header_enums()
    A = ALIGNED
    assert lib.fp8q_quantize_act_1x128(A, 4, 128, A, A, None) in (E["FP8Q_ERR_DEVICE"], E["FP8Q_ERR_LAUNCH"])
    # the fused quantizer with an empty X needs no x / xq / sa
    assert lib.fp8q_quantize_act_w(A, 0, A, 1, 128, 128, 0, 0, A, A, None) == E["FP8Q_ERR_DEVICE"]


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fq.fp8q_quantize_act_1x128(x)


def test_moe_entry_point_argument_checks(lib):
    A = ALIGNED
    E = header_enums()
    d = lib.fp8q_moe_dispatch
    #        ids T  k  e0 E   xq sa K    cap  xs ss off tr rt
    assert d(A, 4, 8, 0, 32, A, A, 100, 32, A, A, A, A, A, None) == E["FP8Q_ERR_SHAPE"]    # K % 128
    assert d(A, 4, 8, 0, 32, A, A, 128, -1, A, A, A, A, A, None) == E["FP8Q_ERR_SHAPE"]    # capacity < 0
    assert d(A, 4, 8, 0, 0, A, A, 128, 32, A, A, A, A, A, None) == E["FP8Q_ERR_SHAPE"]     # E < 1
    assert d(A, 4, 8, 0, 2000, A, A, 128, 32, A, A, A, A, A, None) == E["FP8Q_ERR_SHAPE"]  # E > 1024
    assert d(A, 4, 0, 0, 32, A, A, 128, 32, A, A, A, A, A, None) == E["FP8Q_ERR_SHAPE"]    # k < 1
    assert d(0, 4, 8, 0, 32, A, A, 128, 32, A, A, A, A, A, None) == E["FP8Q_ERR_NULL"]
    assert d(A, 4, 8, 0, 32, A, A, 128, 32, A, A, 0, A, A, None) == E["FP8Q_ERR_NULL"]
    assert d(A + 2, 4, 8, 0, 32, A, A, 128, 32, A, A, A, A, A, None) == E["FP8Q_ERR_ALIGN"]
    assert d(A, 4, 8, 0, 32, A, A + 4, 128, 32, A, A, A, A, A, None) == E["FP8Q_ERR_ALIGN"]
    c = lib.fp8q_moe_combine
    #        out dt cap N   tr wt T  k  y  dt
    assert c(A, 2, 8, 64, A, A, 4, 2, A, 0, None) == E["FP8Q_ERR_DTYPE"]
    assert c(A, 0, 8, 64, A, A, 4, 2, A, 3, None) == E["FP8Q_ERR_DTYPE"]
    assert c(A, 0, 8, 60, A, A, 4, 2, A, 0, None) == E["FP8Q_ERR_SHAPE"]    # N % 8
    assert c(A, 0, 8, 64, A, A, 4, 0, A, 0, None) == E["FP8Q_ERR_SHAPE"]    # k < 1
    assert c(A, 0, 8, 64, A, A, 0, 2, 0, 0, None) == E["FP8Q_OK"]           # no tokens
    assert c(A, 0, 8, 64, 0, A, 4, 2, A, 0, None) == E["FP8Q_ERR_NULL"]
    assert c(A, 0, 8, 64, A, A, 4, 2, A + 2, 0, None) == E["FP8Q_ERR_ALIGN"]


def test_probe_library_exports_and_rejects_bad_arguments():
    """The measurement probes (libfp8q_probe.so, not part of the path) load, export their
    entry points, and reject bad arguments before any HIP call."""
    path = os.path.join(ROOT, "fp8_fine_grained_fp8q_amd", "libfp8q_probe.so")
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    probe = ctypes.CDLL(path)
    for name in ("probe_copy", "probe_read2_write1", "probe_lds_read", "probe_lds_copy", "probe_lds_mix", "probe_mfma"):
        getattr(probe, name).restype = ctypes.c_int
    invalid = 1  # hipErrorInvalidValue
    null = ctypes.c_void_p(0)
    assert probe.probe_copy(null, null, ctypes.c_int64(0), null) == invalid
    assert probe.probe_read2_write1(null, null, ctypes.c_int64(-1), null) == invalid
    assert probe.probe_lds_read(256, 0, null, null, null) == invalid
    assert probe.probe_lds_copy(0, 256, 0, null, null, null, null) == invalid
    assert probe.probe_lds_copy(3, 256, 10, null, null, null, null) == invalid
    assert probe.probe_lds_mix(8, 256, 0, 0, null, null, null, null) == invalid
    assert probe.probe_lds_mix(12, 256, 10, 10, null, null, null, null) == invalid
    assert probe.probe_mfma(5, 256, 10, null, null, null) == invalid
    assert probe.probe_mfma(0, 0, 10, null, null, null) == invalid
