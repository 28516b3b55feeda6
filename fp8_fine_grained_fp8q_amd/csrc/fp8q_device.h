// Device-side helpers shared by the gfx950 kernels of libfp8q: BF16 unpacking, 16-lane
// DPP maximum, the quantizer's correctly rounded division and the E4M3 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// Largest finite E4M3FN magnitude; the online scale is amax / 448.
constexpr float kE4M3Max = 448.0f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (non-temporal hint: read once, do not keep in the caches).
__device__ __forceinline__ uint4 load16_stream(const void *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// The two BF16 values packed in a dword, widened exactly to FP32 (BF16 is the top half
// of an FP32 bit pattern).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Lane `src` of a float held in every lane (readlane is an integer builtin: pass the bits).
__device__ __forceinline__ float lane_f32(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}

// Maximum over the 16 lanes of a DPP row (lanes 16r .. 16r+15), left in every lane of the
// row.  Four rotate-and-max steps (row_ror 8, 4, 2, 1) stay inside the row.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x128, 0xf, 0xf, false));  // row_ror:8
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x124, 0xf, 0xf, false));  // row_ror:4
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x122, 0xf, 0xf, false));  // row_ror:2
  v = fmaxf(v, __builtin_amdgcn_update_dpp(0.0f, v, 0x121, 0xf, 0xf, false));  // row_ror:1
  return v;
}

// Division of the quantizer, y = RN32(x / s), for one group sharing s.
//
// Fast path (s in [2^-64, 2^64]): r = RN(1/s) once per group (IEEE division), then per
// element q0 = RN(x*r) and two residual corrections, each one FMA for the residual and
// one for the update:
//     e1 = RN(x - q0*s),  y1 = RN(q0 + e1*r)      -> y1 is within one ulp of x/s
//     e2 =    x - y1*s (exact),  y = RN(y1 + e2*r) -> y = RN(x/s)
// The second step is Markstein's theorem (IBM J. Res. Dev. 34(1), 1990; see also
// Cornea, Golliver and Markstein, ARITH-14, 1999): with r the correctly rounded
// reciprocal and y1 a faithful quotient, one correction gives the correctly rounded
// quotient, and the residual of a faithful quotient is exactly representable.  The first
// step is needed because q0 alone can be more than one ulp away (r and the product each
// round).  The bounds on s keep every residual clear of underflow whenever
// |x/s| >= 2^-11; smaller quotients become E4M3 zeros whatever their last bits.
// Slow path (any other s > 0): the compiler's IEEE division (correctly rounded; FP32
// denormals are preserved in these kernels).  s == 0 (all-zero group): y = x, i.e. +-0.
struct GroupDiv {
  float s, r;
  int mode;  // 0: zero group, 1: fast, 2: IEEE division
  __device__ __forceinline__ explicit GroupDiv(float scale) : s(scale), r(0.0f), mode(0) {
    if (scale == 0.0f) {
      mode = 0;
    } else if (scale >= 0x1p-64f && scale <= 0x1p64f) {
      mode = 1;
      r = 1.0f / scale;
    } else {
      mode = 2;
    }
  }
  // The correctly rounded fast-path quotient (valid for mode 1 only).  The corrections
  // can turn a zero quotient's sign positive (-0 - (+0) = +0), so the sign of x is put
  // back; the quotient of x by a positive scale always has the sign of x.
  __device__ __forceinline__ float fast(float x) const {
#pragma clang fp contract(off)
    const float q0 = x * r;
    const float e1 = __builtin_fmaf(-q0, s, x);
    const float y1 = __builtin_fmaf(e1, r, q0);
    const float e2 = __builtin_fmaf(-y1, s, x);
    return __builtin_copysignf(__builtin_fmaf(e2, r, y1), x);
  }
  // The same quotient for a dividend with at most 8 significant bits (every BF16 value),
  // mode 1 only: q0 = RN(x*r) and a single correction, y = RN(q0 - e*r) with the residual
  // taken negated, e = RN(q0*s - x).  One correction suffices for such dividends: checked
  // exhaustively for all 128 BF16 significands against all 2^23 FP32 significands of s,
  // every result equal to RN(x/s); the whole computation scales exactly with the exponents
  // of x and s while no intermediate leaves the normal range, which the mode-1 bounds on s
  // ensure for every quotient of magnitude >= 2^-11 (smaller ones are E4M3 zeros).  The
  // negated residual keeps the sign of a zero dividend: x = -0 gives q0 = -0, e = +0 and
  // y = -0 + -0 = -0.  The quotient must be finite: |x/s| stays far below the FP32 range
  // whenever s is at least the group's amax / 448.
  __device__ __forceinline__ float fast_bf16(float x) const {
#pragma clang fp contract(off)
    const float q0 = x * r;
    const float en = __builtin_fmaf(q0, s, -x);
    return __builtin_fmaf(-en, r, q0);
  }
};

// Saturate to the E4M3 range (keeps -0), then pack four FP32 values into four E4M3 bytes
// (element 0 in the low byte) with gfx950's OCP-FP8 conversion (round to nearest even).
__device__ __forceinline__ float sat448(float y) { return __builtin_amdgcn_fmed3f(y, -kE4M3Max, kE4M3Max); }

__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
  return static_cast<uint32_t>(w);
}

// Eight BF16 values (one 16-byte chunk) -> eight E4M3 codes (8 bytes) with divisor `dv`.
// One branch per chunk on the group's division mode (uniform across a group's lanes).
__device__ __forceinline__ uint2 quant8(const uint4 v, const GroupDiv &dv) {
  float y[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  if (dv.mode == 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = dv.fast_bf16(y[i]);
  } else if (dv.mode == 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = y[i] / dv.s;
  }
  uint2 out;
  out.x = pack4_e4m3(y[0], y[1], y[2], y[3]);
  out.y = pack4_e4m3(y[4], y[5], y[6], y[7]);
  return out;
}

// Eight FP32 values -> eight E4M3 codes with divisor `dv` (as quant8, for values held as
// FP32: kBf16Values when each is a widened BF16 value, else any FP32 value, e.g. a fused
// producer's output, which takes the two-correction division).
template <bool kBf16Values>
__device__ __forceinline__ uint2 quant8f(const float (&x)[8], const GroupDiv &dv) {
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = x[i];
  if (dv.mode == 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = kBf16Values ? dv.fast_bf16(y[i]) : dv.fast(y[i]);
  } else if (dv.mode == 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = y[i] / dv.s;
  }
  uint2 out;
  out.x = pack4_e4m3(y[0], y[1], y[2], y[3]);
  out.y = pack4_e4m3(y[4], y[5], y[6], y[7]);
  return out;
}

// Largest |x| of the eight BF16 values in a 16-byte chunk.
__device__ __forceinline__ float absmax8(const uint4 v) {
  float m = fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x)));
  m = fmaxf(m, fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y))));
  m = fmaxf(m, fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))));
  m = fmaxf(m, fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w))));
  return m;
}

}  // namespace fp8q
