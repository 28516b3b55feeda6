// Block-scaled FP8 GEMM for gfx950 (CDNA4), dense and grouped (MoE experts).
//
//   C[m][n] = sum_kb (sa[kb][m] * sb[n/128][kb]) * P_kb[m][n],
//   P_kb[m][n] = sum_{k in block kb} e4m3(xq[m][k]) * e4m3(wq[n][k])
//
// FP8 tensors in, BF16 or FP32 out (dtcms.com DeepSeek-V3 page, section 3.1); partial
// sums leave the matrix units and are accumulated in FP32 registers at every 128-wide K
// block, where the 1x128 activation and 128x128 weight scales apply (codingmall.com page
// on FP8 in DeepSeek-V3 training, section "Tang do chinh xac tich luy"; risenshineclean.com
// training-algorithm page, section 3, "accumulation precision").  On gfx950 one
// v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-wide K block of a 16x16 output tile,
// so each MFMA result is a complete block partial P_kb: it starts from C = 0 and is folded
// into the FP32 accumulator with one FMA per element, acc = P * (sa*sb) + acc.  Those FMAs
// run on the vector ALU one fragment column behind the MFMAs, so the matrix core is never
// waiting on them.
//
// Workgroup tile 256(M) x BN(N) with BN = 32*NFR, K step 128 (= the scale block), 8 waves
// in a 4(M) x 2(N) grid, each owning 64 x 16*NFR outputs (4*NFR*4 FP32 accumulator VGPRs).
// Dense problems use 256-wide tiles, or a column split into a 256-wide range followed by a
// 192-wide range in the same launch when that fills the GPU's CUs in fewer rounds.  The MFMA
// takes the weight fragment as its A operand and the activation fragment as B, so every
// lane owns one output row m and four consecutive columns n: one activation scale per
// fragment row and 8- or 16-byte output stores.
//
// Operand staging: both stages live in LDS, double buffered.  gfx950's buffer_load ... lds
// moves 16 B per lane from global memory straight into LDS, lane p's bytes landing at 16p
// of a 1 KB block, from any global address; each group of 8 lanes fetches one 128-byte
// K block of one row.  Layout of a stage, per group of 16 rows (2 KB): rows r and r+8 of
// the group share a 256-byte line (r in the low half, r+8 in the high half), and the
// 16-byte chunks of a row are XOR-swizzled by r mod 8.  A fragment read (ds_read_b128,
// lane 16kg+r taking chunk 2kg+h of row r) then has lanes 0-7 and 8-15 of each 16-lane
// group in opposite halves of eight different lines at eight different chunk slots; on
// gfx950 this reads at close to the LDS's full 256 B per clock, while a row-major tile
// (two consecutive rows per line) read in fragment shape reaches about half of that
// whatever the swizzle, as the four 16-lane groups then collide on shared lines.  The
// two buffers are separate LDS arrays, so the compiler can see that reading one does not
// wait for the loads in flight into the other.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "fp8q_launch.h"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
#define FP8Q_LDS __attribute__((address_space(3)))

constexpr int kBM = 256;
constexpr int kBK = 128;
constexpr int kThreads = 512;
constexpr int kGroupM = 8;  // M tiles per raster group (L2 reuse of weight panels)

#ifndef FP8Q_PRIO
#define FP8Q_PRIO 1
#endif
// LDS byte offset, within its stage, of chunk c (16 bytes) of row `row` (see above).
__device__ __forceinline__ int lds_pos(int row, int c) {
  const int r = row & 15;
  return (row >> 4) * 2048 + (r & 7) * 256 + (r >> 3) * 128 + ((c ^ (r & 7)) << 4);
}

// Buffer resource (gfx9 family layout) over `bytes` bytes at `p`; loads at or past the
// end return zeros, which is how rows beyond the tile's valid range are filled.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// Per-lane byte offsets of the pieces a lane moves for one stage: wave w fills LDS blocks
// b = 8*i + w (1 KB = 4 lines); lane p of block b lands on line 4*(b%2) + p/16, half
// (p/8)%2, slot p%8 of row group b/2, i.e. on row 16*(b/2) + line + 8*half, chunk
// slot ^ line of that row (the inverse of lds_pos).  Both operands use these offsets (both
// have row stride K).
template <int NO = 4>
__device__ __forceinline__ void stage_offsets(int64_t K, int wave, int lane, uint32_t (&off)[NO]) {
#pragma unroll
  for (int i = 0; i < NO; ++i) {
    const int b = 8 * i + wave;
    const int line = 4 * (b & 1) + (lane >> 4);
    const int row = 16 * (b >> 1) + line + 8 * ((lane >> 3) & 1);
    const int chunk = (lane & 7) ^ line;
    off[i] = static_cast<uint32_t>(row) * static_cast<uint32_t>(K) + static_cast<uint32_t>(chunk << 4);
  }
}

// Copy one stage (K bytes [koff, koff + 128) of 64*NL operand rows) into LDS.  Rows past
// the resource's end (a narrower weight tile, a ragged edge) are filled with zeros by the
// buffer bounds check without touching memory, so every wave always issues NL loads and
// the loop body stays free of branches.
template <int NL = 4>
__device__ __forceinline__ void stage_load(__amdgpu_buffer_rsrc_t rsrc, const uint32_t *off, uint32_t koff,
                                           FP8Q_LDS uint8_t *lds, int wave) {
#pragma unroll
  for (int i = 0; i < NL; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FP8Q_LDS void *)(lds + (8 * i + wave) * 1024), 16,
                                             static_cast<int>(off[i]), static_cast<int>(koff), 0, 0);
}

// One MFMA operand fragment: rows 16g .. 16g+15 of the stage, lane 16kg + r taking K bytes
// [32kg, 32kg + 32) of row 16g + r.  fo0 / fo1 = lds_pos(r, 2kg) / lds_pos(r, 2kg + 1)
// for the lane's r and kg (row group 0).
__device__ __forceinline__ v8i frag(const FP8Q_LDS uint8_t *lds, int g, int fo0, int fo1) {
  const v4i lo = *reinterpret_cast<const FP8Q_LDS v4i *>(lds + g * 2048 + fo0);
  const v4i hi = *reinterpret_cast<const FP8Q_LDS v4i *>(lds + g * 2048 + fo1);
  return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// s_setprio with a value known after unrolling (the builtin needs a literal).
__device__ __forceinline__ void set_prio(int p) {
  switch (p) {
    case 0: __builtin_amdgcn_s_setprio(0); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    default: __builtin_amdgcn_s_setprio(3); break;
  }
}

// Block partial of a 16x16 tile over one 128-wide K block (E4M3 x E4M3, FP32 result).
__device__ __forceinline__ v4f mfma_block(const v8i &a, const v8i &b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

struct Tile {
  int64_t m_begin;  // first row of the tile (global row index)
  int rows;         // valid rows in the tile, 1..256
  int64_t n0;       // first column
  int64_t n_end;    // one past the last column this tile may write
  const uint8_t *x; // activation codes, [M][K]
  const uint8_t *w; // weight matrix of the tile's expert, [N][K]
  const float *sb;  // its block scales, [N/128][K/128]
};

// Dense tile of workgroup `bid` among the tiles of width kBN covering columns
// [n_lo, n_hi) of C.
template <int kBN>
__device__ __forceinline__ void dense_tile(int bid, int64_t M, int64_t n_lo, int64_t n_hi, const uint8_t *wq,
                                           const float *sb, Tile &t) {
  const int tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  const int tiles_n = static_cast<int>((n_hi - n_lo + kBN - 1) / kBN);
  const int total = tiles_m * tiles_n;
  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous run of
  // logical tiles (a bijection on [0, total)) so that its L2 sees neighbouring tiles.
  const int per = total / 8, rem = total % 8;
  const int xcd = bid % 8, idx = bid / 8;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + idx;
  // Raster in groups of kGroupM M-tiles: consecutive tiles share weight / activation panels.
  const int span = kGroupM * tiles_n;
  const int group = logical / span;
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in_group = logical - group * span;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  t.m_begin = static_cast<int64_t>(tm) * kBM;
  t.rows = static_cast<int>(min(static_cast<int64_t>(kBM), M - t.m_begin));
  t.n0 = n_lo + static_cast<int64_t>(tn) * kBN;
  t.n_end = n_hi;
  t.w = wq;
  t.sb = sb;
}

// The LDS stages of one workgroup: activation and weight tiles, double buffered.  Both
// hold 256 rows of one 128-byte K block; narrower weight tiles leave the last rows unused.
struct Stages {
  FP8Q_LDS uint8_t *x0, *w0, *x1, *w1;
  FP8Q_LDS uint8_t *c0, *c1;  // per-column scales of the stage (row-scaled B operand only)
};

// Computes one (64*WM) x (16*NFR*WN) tile of C, WM x WN = 8 waves (4 x 2: 256 x 32*NFR;
// 2 x 4: 128 x 64*NFR), each wave 64 rows x 16*NFR columns.  kRowB: the B operand (t.w)
// carries one scale per row and 128-wide K block, t.sb[K/128][N] (a 1x128 tile quantized
// operand), instead of one per 128x128 block; those scales ride along with each stage
// (1 KB through LDS) and the promotion multiplies the two scales per element.
template <int NFR, bool kRowB = false, int WM = 4>
__device__ __forceinline__ void gemm_tile(const Tile &t, const float *__restrict__ sa, int64_t M, int64_t N,
                                          int64_t K, void *__restrict__ c, int out_f32, const Stages &st) {
  constexpr int WN = 8 / WM;
  constexpr int kBN = 16 * NFR * WN;  // tile columns
  constexpr int kWN = 16 * NFR;       // columns per wave
  constexpr int kXL = WM;             // activation-stage loads per wave (64*WM rows)
  constexpr int kWL = kBN % 64 == 0 ? kBN / 64 : 4;  // weight-stage loads per wave
  constexpr int kNO = kWL > kXL ? kWL : kXL;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;  // rows wm*64 .. +63
  const int wn = wave % WN;  // cols wn*kWN .. +kWN-1
  const int KB = static_cast<int>(K >> 7);
  const int NB = static_cast<int>(N >> 7);
  const int l16 = lane & 15;
  const int kg = lane >> 4;

  // Operand tiles as buffer resources: rows past the valid range read as zeros.
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(t.x + t.m_begin * K, static_cast<uint32_t>(t.rows * K));
  const int rows_w = static_cast<int>(min(static_cast<int64_t>(kBN), t.n_end - t.n0));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(t.w + t.n0 * K, static_cast<uint32_t>(rows_w * K));
  uint32_t off[kNO];
  stage_offsets(K, wave, lane, off);
  const int fo0 = lds_pos(l16, 2 * kg), fo1 = lds_pos(l16, 2 * kg + 1);  // fragment-read offsets
  const int wg0 = wn * kWN / 16;  // first weight row group of this wave

  // activation-scale rows of this lane (one per 16-row fragment), clamped into the tile
  int srow[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int r = wm * 64 + f * 16 + l16;
    srow[f] = static_cast<int>(t.m_begin) + (r < t.rows ? r : t.rows - 1);
  }
  // Weight-block scales: the wave's columns start in 128-column block nb0; fragment
  // columns j >= jsplit lie in block nb0 + 1 (a wave spans at most two blocks).
  const int64_t wc0 = t.n0 + wn * kWN;
  const int nb0 = static_cast<int>(min(static_cast<int64_t>(NB - 1), wc0 >> 7));
  const int nb1 = min(NB - 1, nb0 + 1);
  const int jsplit = static_cast<int>((128 - (wc0 & 127)) >> 4);
  const float *sbrow0 = t.sb + static_cast<int64_t>(kRowB ? 0 : nb0) * KB;
  const float *sbrow1 = t.sb + static_cast<int64_t>(kRowB ? 0 : nb1) * KB;
  // Row-scaled B: the stage's column scales (lane l copies columns 4l .. 4l+3 of the
  // tile).  Every wave issues the same 1 KB copy to the same LDS words: the writes are
  // identical, and a branch here would split the loop body.  The buffer's range check
  // counts the block's row offset (the scalar offset) too, so the resource spans the rest
  // of the scale matrix; the copies past the tile's last column read other columns'
  // finite scales, which only ever meet zero partials.
  const __amdgpu_buffer_rsrc_t rsc = make_rsrc(t.sb + t.n0, static_cast<uint32_t>((KB * N - t.n0) * 4));
  auto scale_load = [&](int kb, FP8Q_LDS uint8_t *dst) {
    if (kRowB)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (FP8Q_LDS void *)dst, 16, lane * 16,
                                               static_cast<int>(kb * N * 4), 0, 0);
  };

  v4f acc[4][NFR];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int j = 0; j < NFR; ++j) acc[f][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  float sa_cur[4], sa_nxt[4];
  float sb0_cur, sb1_cur, sb0_nxt = 0.0f, sb1_nxt = 0.0f;

  stage_load<kXL>(rx, off, 0, st.x0, wave);
  stage_load<kWL>(rw, off, 0, st.w0, wave);
  scale_load(0, st.c0);
#pragma unroll
  for (int f = 0; f < 4; ++f) sa_cur[f] = sa[srow[f]];
  sb0_cur = kRowB ? 0.0f : sbrow0[0];
  sb1_cur = kRowB ? 0.0f : sbrow1[0];
#pragma unroll
  for (int f = 0; f < 4; ++f) sa_nxt[f] = 0.0f;

  // One K block: wait for its stage, start the copy of the next one into the other
  // buffer, then 4*NFR MFMAs (one per 16x16 fragment pair).  The promotion is software
  // pipelined: the block partials of fragment column j are folded into the accumulator
  // (one FMA per element with that row's scale sa*sb) while the MFMAs of column j+1 run;
  // the last column's partials are folded during the next block's first column.  The
  // body is branch-free (at the last block the copy just repeats that block).
  v4f pp[4];      // partials waiting to be folded
  float sclp[4];  // scales of the previous block's last column
  float sa_prev[4];                          // row-scaled B: row scales of the previous block
  v4f sbc_prev = v4f{0.0f, 0.0f, 0.0f, 0.0f};  // row-scaled B: scales of the column being folded
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    pp[f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    sclp[f] = 0.0f;
    sa_prev[f] = 0.0f;
  }
  // kOne (block-scaled B only): all of this wave's columns lie in one 128-column scale
  // block, so a fragment's scale is the same for every column of the step: sa*sb is
  // formed once per step instead of once per column.
  auto step = [&](auto one_block, const FP8Q_LDS uint8_t *cx, const FP8Q_LDS uint8_t *cw, FP8Q_LDS uint8_t *nx,
                  FP8Q_LDS uint8_t *nw, const FP8Q_LDS uint8_t *csc, FP8Q_LDS uint8_t *nsc, int kb) {
    constexpr bool kOne = decltype(one_block)::value;
    float scl0[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) scl0[f] = kOne ? sa_cur[f] * sb0_cur : 0.0f;
    // Stage kb has landed in LDS once every wave's own copies are done (vmcnt(0) before
    // the barrier: the compiler's fence does not count direct-to-LDS loads), and after
    // the barrier every wave is also done reading the other buffer.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // Operands of the first MFMA first, then the copies of the next stage, then the other
    // activation fragments.
    v8i wnext = frag(cw, wg0, fo0, fo1);
    v8i xf[4];
    xf[0] = frag(cx, wm * 4, fo0, fo1);
    const int kn = kb + 1 < KB ? kb + 1 : kb;
    const uint32_t koff = static_cast<uint32_t>(kn) * kBK;
    stage_load<kXL>(rx, off, koff, nx, wave);
    stage_load<kWL>(rw, off, koff, nw, wave);
    scale_load(kn, nsc);
    const float *sak = sa + static_cast<int64_t>(kn) * M;
#pragma unroll
    for (int f = 0; f < 4; ++f) sa_nxt[f] = sak[srow[f]];
    if (!kRowB) {
      sb0_nxt = sbrow0[kn];
      sb1_nxt = sbrow1[kn];
    }
#pragma unroll
    for (int f = 1; f < 4; ++f) xf[f] = frag(cx, wm * 4 + f, fo0, fo1);
#pragma unroll
    for (int j = 0; j < NFR; ++j) {
#if FP8Q_PRIO
      // Progress-based issue priority: the two waves sharing a SIMD compete for its matrix
      // core, and by default the older one wins every time and runs ahead, leaving the
      // younger one alone (and the matrix core under-fed) before each barrier.  Lowering
      // the priority as a wave moves through the block lets the one behind catch up.
      if (j == 0 || (j * 4) / NFR != ((j - 1) * 4) / NFR) set_prio(3 - (j * 4) / NFR);
#endif
      const v8i wf = wnext;
      if (j + 1 < NFR) wnext = frag(cw, wg0 + j + 1, fo0, fo1);
      v4f np[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) np[f] = mfma_block(wf, xf[f]);
      const int jp = j == 0 ? NFR - 1 : j - 1;
      if constexpr (kRowB) {
        // this column's four scales, folded with its partials at the next column
        const v4f sbc_new = *reinterpret_cast<const FP8Q_LDS v4f *>(csc + (wn * kWN + j * 16 + 4 * kg) * 4);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const float sr = j == 0 ? sa_prev[f] : sa_cur[f];
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[f][jp][i] = __builtin_fmaf(pp[f][i] * sbc_prev[i], sr, acc[f][jp][i]);
          pp[f] = np[f];
        }
        sbc_prev = sbc_new;
      } else {
        const float sbj = jp < jsplit ? sb0_cur : sb1_cur;  // wave-uniform
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const float sc = j == 0 ? sclp[f] : (kOne ? scl0[f] : sa_cur[f] * sbj);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[f][jp][i] = __builtin_fmaf(pp[f][i], sc, acc[f][jp][i]);
          pp[f] = np[f];
        }
      }
      // Issue order within a column: each MFMA follows a group of promotion FMAs of the
      // previous column, so the vector ALU work sits between the matrix instructions.
      if constexpr (!kRowB) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // 5 VALU
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const float sbl = NFR - 1 < jsplit ? sb0_cur : sb1_cur;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      sclp[f] = sa_cur[f] * sbl;
      sa_prev[f] = sa_cur[f];
      sa_cur[f] = sa_nxt[f];
    }
    sb0_cur = sb0_nxt;
    sb1_cur = sb1_nxt;
  };

  auto kloop = [&](auto one_block) {
    int kb = 0;
    for (; kb + 1 < KB; kb += 2) {
      step(one_block, st.x0, st.w0, st.x1, st.w1, st.c0, st.c1, kb);
      step(one_block, st.x1, st.w1, st.x0, st.w0, st.c1, st.c0, kb + 1);
    }
    if (kb < KB) step(one_block, st.x0, st.w0, st.x1, st.w1, st.c0, st.c1, kb);
  };
  if (!kRowB && jsplit >= NFR)
    kloop(std::integral_constant<bool, !kRowB>{});
  else
    kloop(std::false_type{});
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the last (repeated) copy
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i)  // the same operation order as the folds inside the loop
      acc[f][NFR - 1][i] = kRowB ? __builtin_fmaf(pp[f][i] * sbc_prev[i], sa_prev[f], acc[f][NFR - 1][i])
                                 : __builtin_fmaf(pp[f][i], sclp[f], acc[f][NFR - 1][i]);

  // Epilogue: lane owns row m = m_begin + wm*64 + f*16 + l16 and columns
  // n0 + wn*kWN + j*16 + 4*kg + {0..3}.
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int r = wm * 64 + f * 16 + l16;
    if (r >= t.rows) continue;
    const int64_t m = t.m_begin + r;
#pragma unroll
    for (int j = 0; j < NFR; ++j) {
      const int64_t n = wc0 + j * 16 + 4 * kg;
      if (n >= t.n_end) continue;
      const v4f v = acc[f][j];
      if (out_f32) {
        *reinterpret_cast<v4f *>(static_cast<float *>(c) + m * N + n) = v;
      } else {
        uint32_t b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t u = __float_as_uint(v[i]);
          b[i] = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;  // round to nearest even
        }
        uint2 pk;
        pk.x = b[0] | (b[1] << 16);
        pk.y = b[2] | (b[3] << 16);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(c) + m * N + n) = pk;
      }
    }
  }
}

#define FP8Q_DECLARE_STAGES(st, scale_bytes)                             \
  __shared__ __attribute__((aligned(1024))) uint8_t sx0[kBM * kBK];      \
  __shared__ __attribute__((aligned(1024))) uint8_t sw0[kBM * kBK];      \
  __shared__ __attribute__((aligned(1024))) uint8_t sx1[kBM * kBK];      \
  __shared__ __attribute__((aligned(1024))) uint8_t sw1[kBM * kBK];      \
  __shared__ __attribute__((aligned(16))) uint8_t sc0[scale_bytes];      \
  __shared__ __attribute__((aligned(16))) uint8_t sc1[scale_bytes];      \
  const Stages st = {(FP8Q_LDS uint8_t *)sx0, (FP8Q_LDS uint8_t *)sw0,   \
                     (FP8Q_LDS uint8_t *)sx1, (FP8Q_LDS uint8_t *)sw1,   \
                     (FP8Q_LDS uint8_t *)sc0, (FP8Q_LDS uint8_t *)sc1}

// Dense problem in two column ranges of different tile widths, one launch: tiles
// [0, tiles1) cover columns [0, n_split) with 32*NFR1-wide tiles, the rest cover
// [n_split, N) with 32*NFR2-wide tiles (tiles1 == total: one width throughout).  Tiles are
// taken in index order, so the wide tiles take the first round and the narrow ones fill
// what would otherwise be a partly idle last round.
//
// Persistent: the grid has at most one workgroup per CU and workgroup b takes tiles b,
// b + gridDim.x, ... (a multiple of 8 keeps every tile on the XCD the mapping assigns it),
// so a CU starts its next tile's copies while the previous tile's output stores drain,
// instead of retiring the workgroup and launching a new one.
//
// kRowB: the B operand carries 1x128 row-tile scales sb[K/128][N] (the weight-gradient GEMM
// over token tiles) instead of 128x128 block scales.
template <int NFR1, int NFR2, bool kRowB = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_blockscaled_split_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ sa, const uint8_t *__restrict__ wq,
    const float *__restrict__ sb, int64_t M, int64_t N, int64_t K, int64_t n_split, int tiles1, int total,
    void *__restrict__ c, int out_f32) {
  FP8Q_DECLARE_STAGES(st, kRowB ? 1024 : 16);
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    Tile t;
    if (item < tiles1) {
      dense_tile<32 * NFR1>(item, M, 0, n_split, wq, sb, t);
      t.x = xq;
      gemm_tile<NFR1, kRowB>(t, sa, M, N, K, c, out_f32, st);
    } else {
      dense_tile<32 * NFR2>(item - tiles1, M, n_split, N, wq, sb, t);
      t.x = xq;
      gemm_tile<NFR2, kRowB>(t, sa, M, N, K, c, out_f32, st);
    }
    // Every wave is past its last LDS read (its data fed the MFMAs) before the next tile's
    // first copy overwrites the stage buffers.  A bare barrier: no wait for the stores.
    __builtin_amdgcn_s_barrier();
  }
}

// Grouped GEMM work items.  Expert g (rows offsets[g] .. offsets[g+1]-1, clamped to
// [0, M_tot)) is cut into floor(n_g / 256) full 256-row tiles, each covering N in 256-wide
// tiles, plus its tail of n_g mod 256 rows: a tail of at most 128 rows uses 128 x 512 tiles
// (the same per-wave work, half as many tiles as 256 x 256 ones would need), a longer tail
// one more row of 256 x 256 tiles.  Items are numbered expert by expert, N tile by N tile,
// M tile last (tiles of one expert sharing a weight panel are adjacent), and workgroups are
// dealt to the 8 XCDs in contiguous runs of items.  Returns the tile shape (0: 256 x 256,
// 1: 128 x 512) or -1 past the last item.
// A value the caller knows to be equal in every lane, moved to a scalar register (so tile
// coordinates derived from lane shuffles still address the operands through SGPRs).
__device__ __forceinline__ int uniform32(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d);
    v += lane >= d ? u : 0;
  }
  return v;
}

__device__ __forceinline__ int grouped_item(const int32_t *__restrict__ offsets, int G, int64_t M_tot, int64_t N,
                                            int64_t K, const uint8_t *wq, const float *sb, Tile &t) {
  const int nt_a = static_cast<int>((N + 255) / 256);
  const int nt_b = static_cast<int>((N + 511) / 512);
  const int lane = threadIdx.x & 63;
  // Expert g's clamped row range [a, b) and its number of work items (lanes past G: 0).
  auto expert = [&](int g, int64_t &a, int64_t &b) -> int {
    a = 0;
    b = 0;
    if (g >= G) return 0;
    a = offsets[g];
    b = offsets[g + 1];
    a = a < 0 ? 0 : (a > M_tot ? M_tot : a);
    b = b < a ? a : (b > M_tot ? M_tot : b);
    const int64_t n = b - a, full = n / 256, tail = n % 256;
    return static_cast<int>(full * nt_a + (tail == 0 ? 0 : (tail <= 128 ? nt_b : nt_a)));
  };
  // The experts are scanned 64 at a time, one per lane (the grid bound keeps every count
  // and the total below 2^31).
  int total = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    int64_t a, b;
    total += __shfl(wave_inclusive_sum(expert(g0 + lane, a, b)), 63);
  }
  total = uniform32(total);
  const int bid = blockIdx.x;
  if (bid >= total) return -1;
  const int per = total / 8, rem = total % 8;
  const int xcd = bid % 8, idx = bid / 8;
  const int item = xcd * per + (xcd < rem ? xcd : rem) + idx;
  int before = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    int64_t a, b;
    const int cnt = expert(g0 + lane, a, b);
    const int incl = wave_inclusive_sum(cnt);
    const int chunk = uniform32(__shfl(incl, 63));
    if (item < before + chunk) {  // wave-uniform: the expert is in this chunk
      const int gl = uniform32(__ffsll(static_cast<unsigned long long>(__ballot(before + incl > item))) - 1);
      const int g = g0 + gl;
      const int64_t ga = uniform64(__shfl(a, gl)), gb = uniform64(__shfl(b, gl));
      int64_t it = uniform64(item - before - (__shfl(incl, gl) - __shfl(cnt, gl)));
      t.w = wq + static_cast<int64_t>(g) * N * K;
      t.sb = sb + static_cast<int64_t>(g) * (N / 128) * (K / 128);
      t.n_end = N;
      const int64_t n = gb - ga, full = n / 256;
      if (it < full * nt_a) {
        t.m_begin = ga + (it % full) * 256;
        t.rows = 256;
        t.n0 = (it / full) * 256;
        return 0;
      }
      it -= full * nt_a;
      t.m_begin = ga + full * 256;
      t.rows = static_cast<int>(n - full * 256);
      if (t.rows <= 128) {
        t.n0 = it * 512;
        return 1;
      }
      t.n0 = it * 256;
      return 0;
    }
    before += chunk;
  }
  return -1;
}

// Grouped GEMM with both tile shapes in one launch; the two 80 KB LDS halves hold one stage
// each (activation rows first, then weight rows), which fits either shape.
__global__ __launch_bounds__(kThreads, 1) void gemm_grouped_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ sa, const uint8_t *__restrict__ wq,
    const float *__restrict__ sb, const int32_t *__restrict__ offsets, int G, int64_t M, int64_t N,
    int64_t K, void *__restrict__ c, int out_f32) {
  constexpr int kHalf = 80 * 1024;
  __shared__ __attribute__((aligned(1024))) uint8_t sbuf0[kHalf];
  __shared__ __attribute__((aligned(1024))) uint8_t sbuf1[kHalf];
  FP8Q_LDS uint8_t *b0 = (FP8Q_LDS uint8_t *)sbuf0;
  FP8Q_LDS uint8_t *b1 = (FP8Q_LDS uint8_t *)sbuf1;
  Tile t;
  const int shape = grouped_item(offsets, G, M, N, K, wq, sb, t);
  if (shape < 0) return;
  t.x = xq;
  if (shape == 0) {
    const Stages st = {b0, b0 + 256 * kBK, b1, b1 + 256 * kBK, nullptr, nullptr};
    gemm_tile<8, false, 4>(t, sa, M, N, K, c, out_f32, st);
  } else {
    const Stages st = {b0, b0 + 128 * kBK, b1, b1 + 128 * kBK, nullptr, nullptr};
    gemm_tile<8, false, 2>(t, sa, M, N, K, c, out_f32, st);
  }
}

// Debug check of the grouped GEMM's offsets: one workgroup scans offsets[0..G] and raises
// a per-device flag on the first violation it sees (plain stores of the same value).
__device__ int32_t g_offsets_bad;

__global__ void offsets_flag_clear_kernel() {
  if (threadIdx.x == 0) g_offsets_bad = 0;
}

__global__ __launch_bounds__(256) void offsets_check_kernel(const int32_t *__restrict__ offsets, int64_t G,
                                                            int64_t M_tot) {
  bool bad = false;
  for (int64_t g = threadIdx.x; g <= G; g += blockDim.x) {
    const int64_t v = offsets[g];
    if (g == 0 && v != 0) bad = true;
    if (g == G && v != M_tot) bad = true;
    if (g > 0 && offsets[g - 1] > v) bad = true;
  }
  if (bad) g_offsets_bad = 1;
}

hipError_t check_grouped_offsets(const int32_t *offsets, int64_t G, int64_t M_tot, hipStream_t stream,
                                 bool *bad) {
  hipLaunchKernelGGL(offsets_flag_clear_kernel, dim3(1), dim3(64), 0, stream);
  hipLaunchKernelGGL(offsets_check_kernel, dim3(1), dim3(256), 0, stream, offsets, G, M_tot);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
  int32_t flag = 0;
  if ((e = hipMemcpyFromSymbol(&flag, HIP_SYMBOL(g_offsets_bad), sizeof(flag), 0, hipMemcpyDeviceToHost)) !=
      hipSuccess)
    return e;
  *bad = flag != 0;
  return hipSuccess;
}

namespace {

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

#ifndef FP8Q_NARROW_COST
#define FP8Q_NARROW_COST 0.82
#endif

// Finish time of `n1` tiles of cost 1 followed by `n2` tiles of cost c2 when each tile
// goes, in order, to the first of `cus` CUs that becomes free.  After the first kind the
// CUs' free times take two values, so the simulation walks two classes of CUs.
double makespan(int64_t n1, int64_t n2, double c2, int64_t cus) {
  const int64_t f = n1 / cus, r = n1 % cus;
  double end = static_cast<double>(f + (r ? 1 : 0));
  double t[2] = {static_cast<double>(f), static_cast<double>(f + 1)};
  const int64_t cnt[2] = {cus - r, r};
  for (int64_t left = n2; left > 0;) {
    const int i = (cnt[1] == 0 || (cnt[0] > 0 && t[0] <= t[1])) ? 0 : 1;
    left -= min(left, cnt[i]);
    end = t[i] + c2 > end ? t[i] + c2 : end;
    t[i] += c2;
  }
  return end;
}

}  // namespace

#ifndef FP8Q_SPLIT
#define FP8Q_SPLIT 1
#endif
#ifndef FP8Q_PERSISTENT
#define FP8Q_PERSISTENT 1
#endif

namespace {

// Tile plan of a dense problem: uniform 256-wide tiles (t2 == 0, n_split == N), or the
// first a*256 columns in 256-wide tiles and the rest in 192-wide ones, whichever finishes
// first by the cost model (a 192-wide tile costs FP8Q_NARROW_COST of a 256-wide one).
// FP8Q_DENSE_SPLIT overrides the choice (for tests): "off" = uniform, an integer a >= 0 =
// split after a*256 columns (clamped below N).
struct Plan {
  int64_t t1, t2, n_split;
};

Plan dense_plan(int64_t M, int64_t N, int64_t cus) {
  const int64_t tm = (M + kBM - 1) / kBM;
  const int64_t tiles = tm * ((N + 255) / 256);
  double best = makespan(tiles, 0, 0.0, cus);
  int64_t best_a = -1;
  const char *force = getenv("FP8Q_DENSE_SPLIT");
  if (force && force[0] && strcmp(force, "auto") != 0) {
    if (strcmp(force, "off") != 0) {
      const long long a = atoll(force);
      best_a = a < 0 ? 0 : (a * 256 < N ? a : (N - 1) / 256);
    }
  } else if (FP8Q_SPLIT && tiles <= 8 * cus) {
    // Past a few rounds the idle part of the last round is a small share of the run.
    for (int64_t a = 0; a * 256 < N; ++a) {
      const int64_t n2 = tm * ((N - a * 256 + 191) / 192);
      const double ms = makespan(tm * a, n2, FP8Q_NARROW_COST, cus);
      if (ms < best * 0.97) {
        best = ms;
        best_a = a;
      }
    }
  }
  if (best_a < 0) return {tiles, 0, N};
  return {tm * best_a, tm * ((N - best_a * 256 + 191) / 192), best_a * 256};
}

template <bool kRowB>
hipError_t launch_dense(const uint8_t *xq, const float *sa, const uint8_t *wq, const float *sb, int64_t M,
                        int64_t N, int64_t K, void *c, bool out_f32, hipStream_t stream) {
  const int64_t cus = device_cus();
  const int64_t tm = (M + kBM - 1) / kBM;
  if (tm * ((N + 191) / 192) > 0x7fffffff) return hipErrorInvalidValue;
  const Plan p = dense_plan(M, N, cus);
  const int64_t total = p.t1 + p.t2;
  const int64_t grid = FP8Q_PERSISTENT ? min(total, (cus / 8) * 8 > 0 ? (cus / 8) * 8 : cus) : total;
  hipLaunchKernelGGL((gemm_blockscaled_split_kernel<8, 6, kRowB>), dim3(static_cast<uint32_t>(grid)),
                     dim3(kThreads), 0, stream, xq, sa, wq, sb, M, N, K, p.n_split, static_cast<int>(p.t1),
                     static_cast<int>(total), c, out_f32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t *xq, const float *sa, const uint8_t *wq, const float *sb,
                       int64_t M, int64_t N, int64_t K, void *c, bool out_f32, hipStream_t stream) {
  return launch_dense<false>(xq, sa, wq, sb, M, N, K, c, out_f32, stream);
}

hipError_t launch_gemm_rowscaled(const uint8_t *aq, const float *sa, const uint8_t *bq, const float *sb,
                                 int64_t M, int64_t N, int64_t K, void *c, bool out_f32, hipStream_t stream) {
  return launch_dense<true>(aq, sa, bq, sb, M, N, K, c, out_f32, stream);
}

hipError_t launch_grouped_gemm(const uint8_t *xq, const float *sa, const uint8_t *wq, const float *sb,
                               const int32_t *offsets, int64_t G, int64_t M_tot, int64_t N, int64_t K,
                               void *c, bool out_f32, hipStream_t stream) {
  // Upper bound on sum_g ceil(n_g / 256) without reading the offsets on the host.
  const int64_t slots = (M_tot + kBM - 1) / kBM + G;
  const int64_t tiles_n = (N + 255) / 256;
  if (slots * tiles_n > 0x7fffffff - 4096 || G > 0x7fffffff) return hipErrorInvalidValue;  // item indices stay in int
  // Upper bound on the number of work items (sum over experts of ceil(n_g/256) rows of
  // 256-wide tiles) without reading the offsets on the host; surplus workgroups exit.
  hipLaunchKernelGGL(gemm_grouped_kernel, dim3(static_cast<uint32_t>(slots * tiles_n)), dim3(kThreads), 0, stream,
                     xq, sa, wq, sb, offsets, static_cast<int>(G), M_tot, N, K, c, out_f32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace fp8q
