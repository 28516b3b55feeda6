"""CPU oracle for online fine-grained FP8 quantization and the block-scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
load anything in this package: only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark do.  It shares no code with the HIP library
and never imports it.

What it follows (page titles and sections of the DeepSeek-V3 pages it is
written from):

* "DeepSeek-V3 ... FP8 mixed-precision training" (dtcms.com), section 3.2
  (fine-grained quantization) and the codingmall.com page on the role of FP8
  precision in DeepSeek-V3's training, section "Dinh luong hat min"
  (fine-grained quantization): activations are grouped and scaled per 1x128
  tile (one token, 128 channels), weights per 128x128 block, each group with
  its own scale.
* codingmall.com, section "Dinh luong truc tuyen" (online quantization), and
  the risenshineclean.com DeepSeek training-algorithm page, section 3, bullet
  "online quantization": each tile's / block's scale is computed from its own
  current values when it is used; no history of past maxima is kept.
* codingmall.com, section "Dinh dang E4M3 hop nhat" (unified E4M3 format), and
  risenshineclean.com section 3, bullet "unified E4M3": one FP8 format, E4M3,
  for every GEMM operand.
* dtcms.com, section 3.1 (mixed-precision framework): the FP8 GEMMs take FP8
  tensors and produce BF16 or FP32.
* codingmall.com, section "Tang do chinh xac tich luy" (raising accumulation
  precision), and risenshineclean.com section 3, bullet "accumulation
  precision": partial results are periodically promoted to FP32 registers.
  The oracle does not model the promotion; it computes the exact result that
  promotion approximates (the dequantized product in FP64), see gemm.py.

Readings where the pages are silent are listed in each module's docstring.
Modules:
    e4m3   -- OCP E4M3 (E4M3FN) decode / encode (nearest, ties to even, saturating)
    quant  -- 1x128 activation-tile and 128x128 weight-block online quantizers
    gemm   -- dequantized FP64 GEMM, dense and grouped, and the acceptance bound
    backward -- dgrad / wgrad of a linear layer: transposed weight blocks, 128x1
              token tiles, the GEMM with per-row scales on both operands
    swiglu -- SwiGLU of the expert up-projection output followed by the 1x128 quantizer
    comparators -- tensor-level and delayed (historical-max) scaling, for the accuracy study
    moe    -- expert-parallel dispatch (expert-sorted rows of codes and scales) and combine
"""
from . import e4m3, quant, gemm, backward, swiglu, comparators, moe  # noqa: F401
