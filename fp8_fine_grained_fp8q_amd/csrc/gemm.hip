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
// Two kernels share this layout.  The ping-pong kernel (gemm_tile_pp, the dense default and
// the grouped kernel) has the two waves of each SIMD take turns between LDS reads and
// MFMAs; its tiles are 256 wide and 256 rows tall, or 64/128/192 rows for the grouped
// kernel's expert tails and for a dense problem's last round of tiles.  The split-plan
// kernel (gemm_tile, the row-scaled weight-gradient GEMM) runs one barrier per K step and
// uses 256-wide tiles, or a 256-wide column range followed by a 192-wide one in the same
// launch when that fills the GPU's CUs in fewer rounds.  The MFMA takes the weight
// fragment as its A operand and the activation fragment as B, so every lane owns one
// output row m and four consecutive columns n: one activation scale per fragment row and
// 8- or 16-byte output stores.
//
// Operand staging: the stages live in LDS, double buffered.  gfx950's buffer_load ... lds
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
  // Row-scaled B: the stage's 256 column scales (1 KB).  Waves 0-3 each copy a quarter
  // (4 bytes per lane, columns 64q .. 64q+63 to bytes 256q ..), waves 4-7 issue the same
  // copy through an empty resource (zeros, no memory traffic) into the unread second KB of
  // the 2 KB stage array: every wave issues one copy per stage (no branch in the loop body)
  // and the scales cross the fabric once.  The buffer's range check counts the block's row
  // offset (the scalar offset) too, so the resource spans the rest of the scale matrix; the
  // copies past the tile's last column read other columns' finite scales, which only ever
  // meet zero partials.
  const int sq = wave & 3;
  const __amdgpu_buffer_rsrc_t rsc =
      wave < 4 ? make_rsrc(t.sb + t.n0, static_cast<uint32_t>((KB * N - t.n0) * 4)) : make_rsrc(t.sb, 0u);
  const int sc_dst = (wave < 4 ? 0 : 1024) + sq * 256;
  auto scale_load = [&](int kb, FP8Q_LDS uint8_t *dst) {
    if (kRowB)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (FP8Q_LDS void *)(dst + sc_dst), 4, sq * 256 + lane * 4,
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

// ---------------------------------------------------------------------------------------
// Ping-pong schedule for 256 x 256 tiles.  The two waves that share a SIMD (wave w and
// w + 4) take turns: while one multiplies operands it already holds in registers, the
// other reads its next operands from LDS, and they swap at every workgroup barrier.  The
// waves 0-3 run one phase ahead of the waves 4-7, so in every phase each SIMD has one wave
// feeding its matrix core and the LDS reads never sit between a barrier and the first MFMA.
//
// Each wave owns 16*FM rows (FM = 4 for full 256-row tiles; the grouped kernel also runs
// 64-, 128- and 192-row tiles) x 128 columns.  A K block is four phases for a wave:
//   M0: read the activation fragments (FM row groups) and the weight fragments of its
//       column half 0 (fragment columns 0-3),
//   C0: 4*FM MFMAs (FM x 4 fragments) with the promotion FMAs in their shadow,
//   M1: read the weight fragments of column half 1 (fragment columns 4-7),
//   C1: 4*FM MFMAs and promotion.
// The LDS stage is split into three regions: X (activation rows), W0 (the weight rows of
// column half 0 of both wave columns) and W1 (half 1).  X and W0 are read only in M0
// phases and W1 only in M1 phases, so with two buffers each region is free two phases after
// its last read and its next copy (two K blocks ahead) gets about one and a half K blocks
// of time to land: the copies of X and W0 for block kb + 2 are issued in M1(kb), those of
// W1 for block kb + 1 in M0(kb), with the activation scales of block kb + 1.  Per K block a
// wave issues a fixed number of vector memory operations in a fixed order (with the 4 x 2
// wave grid: FM + 2 copies of X/W0, 2 of W1, FM scale loads), so fixed vmcnt counts name exactly
// the copies that must have landed before the barrier preceding their first read.
// Copies past the last K block read through an empty buffer resource (zeros, no memory
// traffic) and keep the counts uniform.  Every wave waits for its own copies at the end of
// its M phases (the loop body has no branch: a branch there lets the compiler move the
// promotion FMAs out of the MFMA phases).
// ---------------------------------------------------------------------------------------
struct PPStages {
  FP8Q_LDS uint8_t *x[2];   // 32 KB each: 256 activation rows
  FP8Q_LDS uint8_t *w0[2];  // 16 KB each: weight rows of column half 0
  FP8Q_LDS uint8_t *w1[2];  // 16 KB each: column half 1
};

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Computes the (16 * WM * FM) x (32 * NFR) tile t, NFR = 8 (256 wide) or 7 (224 wide),
// WM = 4 wave rows (or 2 with 4 wave columns), FM = 1..4: each wave owns 16*FM rows x 16*NFR
// columns, C0 covers its fragment columns 0-3 and C1 columns 4 .. NFR-1.
// The weight regions always hold 8 row groups; with NFR = 7 the last group of each wave
// column in W1 is never read and its copies go through the empty resource.  kOne: every
// wave's columns lie in one 128-column weight-scale block (256-wide tiles starting at a
// multiple of 256), so a fragment row has one promotion scale per K block; otherwise each
// fragment column picks the scale of its block.
//
// kVSB (with kOne): the weight-block scale of each K block is fetched with a vector load
// (uniform across the wave) instead of a scalar load.  Scalar loads share their counter
// with the LDS reads, so the barrier's lgkmcnt(0) after every phase would also wait for the
// next block's scale; when that misses in the caches (a grouped tile's expert scales) the
// wait lands on the critical path.  As a vector load it is one more operation in the
// fixed per-block sequence, waited for by the compiler before its use a block later.  (The
// dense kernel keeps the scalar load: its scale rows stay cached, and the vector form
// measured the same there.)
template <int WM, int NFR, bool kOne, int FM = 4, bool kVSB = false>
__device__ __forceinline__ void gemm_tile_pp(const Tile &t, const float *__restrict__ sa, int64_t M, int64_t N,
                                             int64_t K, void *__restrict__ c, int out_f32, const PPStages &st) {
  static_assert(NFR == 7 || NFR == 8, "wave columns 112 or 128");
  static_assert(WM == 4 || (WM == 2 && NFR == 8), "wave grid 4 x 2, or 2 x 4 with 128-column waves");
  static_assert(!kOne || NFR == 8, "one scale block per wave needs 128-column waves");
  static_assert(FM >= 1 && FM <= 4 && (WM * FM) % 4 == 0, "fragment rows per wave 1..4, whole X copies");
  static_assert(!kVSB || kOne, "vector weight-scale loads: one scale block per wave");
  constexpr int WN = 8 / WM;     // wave columns
  constexpr int kWN = 16 * NFR;  // columns per wave
  constexpr int kNC1 = NFR - 4;  // fragment columns of C1
  // vector memory operations per K block: X/W0 copies, W1 copies, activation scales
  constexpr int kXI = WM * FM / 4;  // X copies per wave (64*WM*FM/4 rows, 8 rows per copy and wave)
  constexpr int kXW0 = kXI + WN, kW1 = WN, kSA = FM + (kVSB ? 1 : 0);  // kSA: the block's scale loads
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lead = wave < 4;  // waves 0-3 run one phase ahead
  const int wm = wave / WN;    // rows wm*16*FM .. +16*FM-1
  const int wn = wave % WN;    // cols wn*kWN .. +kWN-1
  const int KB = static_cast<int>(K >> 7);
  const int NB = static_cast<int>(N >> 7);
  const int l16 = lane & 15;
  const int kg = lane >> 4;

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(t.x + t.m_begin * K, static_cast<uint32_t>(t.rows * K));
  const int rows_w = static_cast<int>(min(static_cast<int64_t>(WN * kWN), t.n_end - t.n0));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(t.w + t.n0 * K, static_cast<uint32_t>(rows_w * K));
  const __amdgpu_buffer_rsrc_t rnull = make_rsrc(t.x, 0u);
  // Activation scales of the tile's rows: sa[kb][m_begin + r] at byte kb*M*4 + r*4; rows
  // past the tile read other rows' (finite) scales or zeros, and only meet zero partials.
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(sa + t.m_begin, static_cast<uint32_t>(((KB - 1) * M + t.rows) * 4));

  // Copies: every 1 KB block this wave moves lands on rows rowbase + 16*(block/2) of its
  // region (the stage layout of lds_pos), so one per-lane offset serves all of them; the
  // rest is a scalar offset.  X (64*WM rows): blocks 8i + wave, i < WM, tile rows
  // 64i + rowbase.  Weight region r (64 rows of each of the WN wave columns): blocks
  // 8i + wave, i < WN, region group 4i + wave/2 = rows 16*(wave/2) .. of wave column i,
  // tile rows kWN*i + 64r + rowbase.
  const int line = 4 * (wave & 1) + (lane >> 4);
  const int rowbase = 16 * (wave >> 1) + line + 8 * ((lane >> 3) & 1);
  const int voff = rowbase * static_cast<int>(K) + (((lane & 7) ^ line) << 4);
  const bool w1_pad = (wave >> 1) >= kNC1;  // this wave's W1 blocks are the unused groups
  const int fo0 = lds_pos(l16, 2 * kg), fo1 = lds_pos(l16, 2 * kg + 1);
  const int sa_off = (wm * 16 * FM + l16) * 4;  // + f*64 for fragment row f

  // Weight-block scales: the wave's columns start in block nb0; fragment columns
  // j >= jsplit lie in block nb0 + 1.
  const int64_t wc0 = t.n0 + wn * kWN;
  const int nb0 = static_cast<int>(min(static_cast<int64_t>(NB - 1), wc0 >> 7));
  const int nb1 = min(NB - 1, nb0 + 1);
  const int jsplit = kOne ? NFR : static_cast<int>((128 - (wc0 & 127)) >> 4);
  const float *sbrow0 = t.sb + static_cast<int64_t>(nb0) * KB;
  const float *sbrow1 = t.sb + static_cast<int64_t>(nb1) * KB;

  v4f acc[FM][NFR];
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int j = 0; j < NFR; ++j) acc[f][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // X and W0 of block s into buffer s % 2 (6 loads), W1 of block s (2 loads), the lane's
  // activation scales of block s (4 loads); blocks past the last read zeros / the last.
  const int K32 = static_cast<int>(K);
  auto copy_xw0 = [&](int s, auto buf) {
    constexpr int b = decltype(buf)::value;
    const bool ok = s < KB;
    const __amdgpu_buffer_rsrc_t r_x = ok ? rx : rnull, r_w = ok ? rw : rnull;
    const int koff = ok ? s * kBK : 0;
#pragma unroll
    for (int i = 0; i < kXI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_x, (FP8Q_LDS void *)(st.x[b] + (8 * i + wave) * 1024), 16, voff,
                                               koff + 64 * i * K32, 0, 0);
#pragma unroll
    for (int i = 0; i < WN; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_w, (FP8Q_LDS void *)(st.w0[b] + (8 * i + wave) * 1024), 16, voff,
                                               koff + kWN * i * K32, 0, 0);
  };
  auto copy_w1 = [&](int s, auto buf) {
    constexpr int b = decltype(buf)::value;
    const bool ok = s < KB && !w1_pad;
    const __amdgpu_buffer_rsrc_t r_w = ok ? rw : rnull;
    const int koff = ok ? s * kBK : 0;
#pragma unroll
    for (int i = 0; i < WN; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r_w, (FP8Q_LDS void *)(st.w1[b] + (8 * i + wave) * 1024), 16, voff,
                                               koff + (kWN * i + 64) * K32, 0, 0);
  };
  auto load_sa = [&](int s, float (&dst)[FM]) {
    const int so = (s < KB ? s : KB - 1) * static_cast<int>(M) * 4;
#pragma unroll
    for (int f = 0; f < FM; ++f)
      dst[f] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsa, sa_off + 64 * f, so, 0));
  };
  // kVSB: the weight-block scale of block s (the wave's one scale block), as a vector load
  const __amdgpu_buffer_rsrc_t rsb =
      make_rsrc(kVSB ? static_cast<const void *>(sbrow0) : static_cast<const void *>(t.x),
                kVSB ? static_cast<uint32_t>(KB * 4) : 0u);
  auto load_sb = [&](int s) -> float {
    const int kn = s < KB ? s : KB - 1;
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsb, kn * 4, 0, 0));
  };
  // Phase boundary: this wave's LDS reads are complete (lgkmcnt(0)), then the workgroup
  // barrier.  Written as one asm statement with a memory clobber rather than
  // __syncthreads(), whose workgroup fence would also wait for every direct-to-LDS copy in
  // flight (vmcnt(0)) and so drain the copy pipeline at every phase; the copies' own
  // completion is covered by the vmcnt waits below.  Nothing is scheduled across it: the
  // MFMAs carry no memory dependence and would otherwise drift into the neighbouring phase.
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Keeps the groups of vector memory operations in program order (the vmcnt counts name
  // copies by their position in that order).
  auto vm_order = [&]() { asm volatile("" ::: "memory"); };

  v8i xf[FM], wf[4];
  v4f pp[FM];       // partials of the last fragment column of the previous C phase
  float sclp[FM];   // their scales
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    pp[f] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    sclp[f] = 0.0f;
  }
  float saA[FM], saB[FM];
  float sb0A = kVSB ? 0.0f : sbrow0[0], sb1A = kOne ? 0.0f : sbrow1[0], sb0B = 0.0f, sb1B = 0.0f;
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  // Prologue: X/W0 of block 0, W1 of block 0, scales of block 0, X/W0 of block 1.
  copy_xw0(0, B0{});
  vm_order();
  copy_w1(0, B0{});
  vm_order();
  load_sa(0, saA);
  if constexpr (kVSB) sb0A = load_sb(0);
  vm_order();
  copy_xw0(1, B1{});
  vm_wait<kW1 + kSA + kXW0>();  // X/W0 of block 0 landed (W1 0, the scales, X/W0 1 may be in flight)
  barrier();
  if (!lead) barrier();  // the lagging waves' first phase is idle

  // C phase over fragment columns j0 .. j0+nc-1 with operands xf, wf; sc0 / sc1: this
  // block's promotion scales of the columns before / from jsplit.
  auto cphase = [&](int j0, int nc, const float (&sc0)[FM], const float (&sc1)[FM]) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if (jj >= nc) break;
      const int jp = jj == 0 ? (j0 == 0 ? NFR - 1 : j0 - 1) : j0 + jj - 1;  // column being folded
      const bool first = jp < jsplit;                                       // wave-uniform
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        const float sf = jj == 0 ? sclp[f] : (kOne || first ? sc0[f] : sc1[f]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[f][jp][i] = __builtin_fmaf(pp[f][i], sf, acc[f][jp][i]);
        pp[f] = mfma_block(wf[jj], xf[f]);
      }
#pragma unroll
      for (int q = 0; q < FM; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // 4 VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    const int jl = j0 + nc - 1;  // the column left for the next phase's first fold
#pragma unroll
    for (int f = 0; f < FM; ++f) sclp[f] = kOne || jl < jsplit ? sc0[f] : sc1[f];
  };

  // One K block kb in buffer buf = kb % 2: sac / sb*c its scales, san / sb*n receive block
  // kb + 1's.
  auto kstep = [&](int kb, auto buf, float (&sac)[FM], float (&san)[FM], float &sb0c, float &sb1c, float &sb0n,
                   float &sb1n) {
    constexpr int b = decltype(buf)::value;
    using Next = std::integral_constant<int, 1 - b>;
    // M0: the fragment reads first (ahead of this phase's copies), then the copies of W1
    // for block kb + 1 and the scales of block kb + 1; this block's promotion scales are
    // formed before the barrier so that C0 starts with its first MFMA.
#pragma unroll
    for (int f = 0; f < FM; ++f) xf[f] = frag(st.x[b], wm * FM + f, fo0, fo1);
#pragma unroll
    for (int j = 0; j < 4; ++j) wf[j] = frag(st.w0[b], wn * 4 + j, fo0, fo1);
    vm_order();
    copy_w1(kb + 1, Next{});
    vm_order();
    load_sa(kb + 1, san);
    if constexpr (kVSB) sb0n = load_sb(kb + 1);
    vm_order();
    if constexpr (!kVSB) {
      const int kn = kb + 1 < KB ? kb + 1 : KB - 1;
      sb0n = sbrow0[kn];
      if (!kOne) sb1n = sbrow1[kn];
    }
    // W1 of block kb landed (before phase 4kb+1 ends for either group); issued after it:
    // the scales of kb, X/W0 of kb+1, W1 and the scales of kb+1
    vm_wait<kSA + kXW0 + kW1 + kSA>();
    float sc0[FM], sc1[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      sc0[f] = sac[f] * sb0c;
      sc1[f] = kOne ? sc0[f] : sac[f] * sb1c;
    }
    barrier();
    // C0
    cphase(0, 4, sc0, sc1);
    barrier();
    // M1
#pragma unroll
    for (int j = 0; j < kNC1; ++j) wf[j] = frag(st.w1[b], wn * 4 + j, fo0, fo1);
    vm_order();
    copy_xw0(kb + 2, buf);
    vm_order();
    // X/W0 of block kb + 1 landed; issued after it: W1 and the scales of kb+1, X/W0 of kb+2
    vm_wait<kW1 + kSA + kXW0>();
    barrier();
    // C1
    cphase(4, kNC1, sc0, sc1);
    barrier();
  };

  int kb = 0;
  for (; kb + 1 < KB; kb += 2) {
    kstep(kb, B0{}, saA, saB, sb0A, sb1A, sb0B, sb1B);
    kstep(kb + 1, B1{}, saB, saA, sb0B, sb1B, sb0A, sb1A);
  }
  if (kb < KB) kstep(kb, B0{}, saA, saB, sb0A, sb1A, sb0B, sb1B);
  if (lead) barrier();  // matches the lagging waves' extra first phase
  vm_wait<0>();         // the copies past the last block (empty) and the scale loads
#pragma unroll
  for (int f = 0; f < FM; ++f)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[f][NFR - 1][i] = __builtin_fmaf(pp[f][i], sclp[f], acc[f][NFR - 1][i]);

  // Epilogue (as gemm_tile): lane owns row m = m_begin + wm*16*FM + f*16 + l16 and columns
  // wc0 + j*16 + 4*kg + {0..3}.
#pragma unroll
  for (int f = 0; f < FM; ++f) {
    const int r = wm * 16 * FM + f * 16 + l16;
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
        uint32_t bb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t u = __float_as_uint(v[i]);
          bb[i] = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;  // round to nearest even
        }
        uint2 pk;
        pk.x = bb[0] | (bb[1] << 16);
        pk.y = bb[2] | (bb[3] << 16);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(c) + m * N + n) = pk;
      }
    }
  }
}

// Tile `idx` of the rectangle rows [m_lo, m_hi) x columns [n_lo, n_hi) of C cut into tiles
// of bm rows and 256 columns (m_hi - m_lo a multiple of bm), with dense_tile's XCD-aware
// raster; the rectangle's first tile index must be a multiple of 8 for the XCD runs to
// line up (any index is correct).
__device__ __forceinline__ void region_tile(int idx, int64_t m_lo, int64_t m_hi, int bm, int64_t n_lo,
                                            int64_t n_hi, const uint8_t *wq, const float *sb, Tile &t) {
  const int tiles_m = static_cast<int>((m_hi - m_lo) / bm);
  const int tiles_n = static_cast<int>((n_hi - n_lo + 255) / 256);
  const int total = tiles_m * tiles_n;
  const int per = total / 8, rem = total % 8;
  const int xcd = idx % 8, j = idx / 8;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + j;
  const int span = kGroupM * tiles_n;
  const int group = logical / span;
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in_group = logical - group * span;
  t.m_begin = m_lo + static_cast<int64_t>(first_m + in_group % gm) * bm;
  t.rows = bm;
  t.n0 = n_lo + static_cast<int64_t>(in_group / gm) * 256;
  t.n_end = n_hi;
  t.w = wq;
  t.sb = sb;
}

// Two-region plan of a dense problem (M and N multiples of 256) whose 256 x 256 tiles fill
// q CU rounds and three quarters (or a half, or a quarter) of one more: region B, rows
// [0, rb) x columns [0, cb), is cut into one round of tiles of 64*hb rows, and the rest,
// rows [rb, M) x [0, cb) and all rows x [cb, N), into q whole rounds of 256-row tiles
// (items 0 .. ta-1; region B takes the last round, item ta + b on workgroup b).  The last
// round's tiles then do hb/4 of a full tile's work instead of leaving CUs idle.  Returns the
// item's tile height in units of 64 rows.
__device__ __forceinline__ int plan_tile(int item, int64_t M, int64_t N, int64_t rb, int64_t cb, int hb,
                                         const uint8_t *wq, const float *sb, Tile &t) {
  const int ta1 = static_cast<int>(((M - rb) / 256) * (cb / 256));
  const int ta2 = static_cast<int>((M / 256) * ((N - cb) / 256));
  if (item < ta1) {
    region_tile(item, rb, M, 256, 0, cb, wq, sb, t);
    return 4;
  }
  if (item < ta1 + ta2) {
    region_tile(item - ta1, 0, M, 256, cb, N, wq, sb, t);
    return 4;
  }
  region_tile(item - ta1 - ta2, 0, rb, 64 * hb, 0, cb, wq, sb, t);
  return hb;
}

// Dense problem in 256 x (32*NFR) tiles with the ping-pong schedule, persistent like
// gemm_blockscaled_split_kernel (workgroup b takes tiles b, b + gridDim.x, ...); hb > 0
// selects plan_tile's two-region plan (NFR = 8 only).
template <int NFR>
__global__ __launch_bounds__(kThreads, 1) void gemm_pp_kernel(const uint8_t *__restrict__ xq,
                                                              const float *__restrict__ sa,
                                                              const uint8_t *__restrict__ wq,
                                                              const float *__restrict__ sb, int64_t M, int64_t N,
                                                              int64_t K, int total, void *__restrict__ c,
                                                              int out_f32, int64_t rb, int64_t cb, int hb) {
  __shared__ __attribute__((aligned(1024))) uint8_t sx0[256 * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sx1[256 * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sw00[128 * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sw01[128 * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sw10[128 * kBK];
  __shared__ __attribute__((aligned(1024))) uint8_t sw11[128 * kBK];
  const PPStages st = {{(FP8Q_LDS uint8_t *)sx0, (FP8Q_LDS uint8_t *)sx1},
                       {(FP8Q_LDS uint8_t *)sw00, (FP8Q_LDS uint8_t *)sw01},
                       {(FP8Q_LDS uint8_t *)sw10, (FP8Q_LDS uint8_t *)sw11}};
  // the full tiles (all of them without a plan), then the plan's last round of short tiles
  const int full = hb == 0 ? total : total - static_cast<int>(gridDim.x);
  for (int item = blockIdx.x; item < full; item += gridDim.x) {
    Tile t;
    if (NFR != 8 || hb == 0)
      dense_tile<32 * NFR>(item, M, 0, N, wq, sb, t);
    else
      plan_tile(item, M, N, rb, cb, hb, wq, sb, t);
    t.x = xq;
    gemm_tile_pp<4, NFR, NFR == 8>(t, sa, M, N, K, c, out_f32, st);
    __builtin_amdgcn_s_barrier();
  }
  if constexpr (NFR == 8) {
    if (hb != 0) {
      Tile t;
      plan_tile(full + static_cast<int>(blockIdx.x), M, N, rb, cb, hb, wq, sb, t);
      t.x = xq;
      if (hb == 3)
        gemm_tile_pp<4, 8, true, 3>(t, sa, M, N, K, c, out_f32, st);
      else if (hb == 2)
        gemm_tile_pp<4, 8, true, 2>(t, sa, M, N, K, c, out_f32, st);
      else
        gemm_tile_pp<4, 8, true, 1>(t, sa, M, N, K, c, out_f32, st);
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
  FP8Q_DECLARE_STAGES(st, kRowB ? 2048 : 16);
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

// Grouped work items with balanced tile heights: expert g's n_g rows, in U = ceil(n_g / 64)
// units of 64 rows, are cut into m_g = ceil(U / 4) row tiles whose heights (in units, at
// most 4) differ by at most one: the first U mod m_g tiles get ceil(U / m_g) units, the rest
// floor(U / m_g) (the last tile holds the remainder of the rows).  So no expert computes more
// than 63 padding rows, and the tiles of one expert take about the same time.  Tiles are 256
// columns wide; the m_g tiles of one 256-column weight panel form a group; groups are
// numbered expert by expert, panel by panel (k = g*P + p, P the number of panels), and
// group k runs on XCD k mod 8, its tiles consecutively, so that the
// tiles sharing a weight panel run side by side under one L2 and every XCD gets the same
// mix of tile heights.  Workgroup b runs on XCD b mod 8 and takes item b / 8 of that XCD's
// list.  Returns h (the tile's 16-row fragments per wave) or -1 for a surplus workgroup.
__device__ __forceinline__ int grouped_item(const int32_t *__restrict__ offsets, int G, int64_t M_tot,
                                                 int64_t N, int64_t K, const uint8_t *wq, const float *sb,
                                                 Tile &t) {
  const int P = static_cast<int>((N + 255) / 256);
  const int lane = threadIdx.x & 63;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, idx = bid >> 3;
  // Expert g's clamped row range [a, b), tiles per panel m, its rows in 64-row units u,
  // and its number of items on this XCD (lanes past G: 0).
  auto expert = [&](int g, int64_t &a, int64_t &b, int &m, int &u) -> int {
    a = 0;
    b = 0;
    m = 0;
    u = 0;
    if (g >= G) return 0;
    a = offsets[g];
    b = offsets[g + 1];
    a = a < 0 ? 0 : (a > M_tot ? M_tot : a);
    b = b < a ? a : (b > M_tot ? M_tot : b);
    const int64_t n = b - a;
    if (n == 0) return 0;
    m = static_cast<int>((n + 255) / 256);
    u = static_cast<int>((n + 63) / 64);
    // groups k in [g*P, g*P + P) with k mod 8 == xcd
    const int64_t k0 = static_cast<int64_t>(g) * P;
    const int64_t cnt = (k0 + P - 1 - xcd + 8) / 8 - (k0 - 1 - xcd + 8) / 8;
    return static_cast<int>(cnt * m);
  };
  int before = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    int64_t a, b;
    int m, u;
    const int cnt = expert(g0 + lane, a, b, m, u);
    const int incl = wave_inclusive_sum(cnt);
    const int chunk = uniform32(__shfl(incl, 63));
    if (idx < before + chunk) {  // wave-uniform: the expert is in this chunk
      const int gl = uniform32(__ffsll(static_cast<unsigned long long>(__ballot(before + incl > idx))) - 1);
      const int g = g0 + gl;
      const int64_t ga = uniform64(__shfl(a, gl));
      const int64_t n = uniform64(__shfl(b, gl)) - ga;
      const int mg = uniform32(__shfl(m, gl)), ug = uniform32(__shfl(u, gl));
      const int r = idx - before - (uniform32(__shfl(incl, gl)) - uniform32(__shfl(cnt, gl)));
      const int j = r / mg, i = r % mg;  // j-th group of expert g on this XCD, tile i of it
      const int hq = ug / mg, hr = ug % mg;
      const int hg = hq + (i < hr ? 1 : 0);          // tile i's height in 64-row units
      const int u0 = i * hq + (i < hr ? i : hr);     // its first row, in units
      const int64_t k0 = static_cast<int64_t>(g) * P;
      const int64_t kfirst = k0 + ((xcd - k0 % 8) + 8) % 8;
      const int p = static_cast<int>(kfirst + 8 * j - k0);
      t.w = wq + static_cast<int64_t>(g) * N * K;
      t.sb = sb + static_cast<int64_t>(g) * (N / 128) * (K / 128);
      t.n_end = N;
      t.n0 = static_cast<int64_t>(p) * 256;
      t.m_begin = ga + static_cast<int64_t>(u0) * 64;
      const int64_t left = n - static_cast<int64_t>(u0) * 64;
      t.rows = static_cast<int>(left < 64 * hg ? left : 64 * hg);
      return hg;
    }
    before += chunk;
  }
  return -1;
}

// Grouped GEMM on the ping-pong schedule with 256-column tiles of 64, 128, 192 or 256 rows
// (grouped_item): 16*h rows per wave for h = 1..4, the LDS regions as for dense tiles.
// The expert tails are short tiles rather than padded ones (their time is mostly the weight
// panel's stream, which a taller tile would not shorten).
__global__ __launch_bounds__(kThreads, 1) void gemm_grouped_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ sa, const uint8_t *__restrict__ wq,
    const float *__restrict__ sb, const int32_t *__restrict__ offsets, int G, int64_t M, int64_t N,
    int64_t K, void *__restrict__ c, int out_f32) {
  __shared__ __attribute__((aligned(1024))) uint8_t sx0[32768];
  __shared__ __attribute__((aligned(1024))) uint8_t sx1[32768];
  __shared__ __attribute__((aligned(1024))) uint8_t sw00[16384];
  __shared__ __attribute__((aligned(1024))) uint8_t sw01[16384];
  __shared__ __attribute__((aligned(1024))) uint8_t sw10[16384];
  __shared__ __attribute__((aligned(1024))) uint8_t sw11[16384];
  const PPStages st = {{(FP8Q_LDS uint8_t *)sx0, (FP8Q_LDS uint8_t *)sx1},
                       {(FP8Q_LDS uint8_t *)sw00, (FP8Q_LDS uint8_t *)sw01},
                       {(FP8Q_LDS uint8_t *)sw10, (FP8Q_LDS uint8_t *)sw11}};
  Tile t;
  const int h = grouped_item(offsets, G, M, N, K, wq, sb, t);
  if (h < 0) return;
  t.x = xq;
  switch (h) {
    case 1: gemm_tile_pp<4, 8, true, 1, true>(t, sa, M, N, K, c, out_f32, st); break;
    case 2: gemm_tile_pp<4, 8, true, 2, true>(t, sa, M, N, K, c, out_f32, st); break;
    case 3: gemm_tile_pp<4, 8, true, 3, true>(t, sa, M, N, K, c, out_f32, st); break;
    default: gemm_tile_pp<4, 8, true, 4, true>(t, sa, M, N, K, c, out_f32, st); break;
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

int device_cu_count() {
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

namespace {

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

#ifndef FP8Q_PP
#define FP8Q_PP 1
#endif

// Whether a dense problem runs on the ping-pong kernel: FP8Q_PP by default, overridden by
// the environment variable FP8Q_DENSE_KERNEL ("pp" or "split"); the kernel's 32-bit buffer
// offsets need M * K/128 < 2^30.
bool use_pp(int64_t M, int64_t K) {
  bool pp = FP8Q_PP != 0;
  const char *e = getenv("FP8Q_DENSE_KERNEL");
  if (e && strcmp(e, "pp") == 0) pp = true;
  if (e && strcmp(e, "split") == 0) pp = false;
  return pp && M * (K / 128) < (static_cast<int64_t>(1) << 30);
}

template <bool kRowB>
hipError_t launch_dense(const uint8_t *xq, const float *sa, const uint8_t *wq, const float *sb, int64_t M,
                        int64_t N, int64_t K, void *c, bool out_f32, hipStream_t stream) {
  const int64_t cus = device_cu_count();
  if (!kRowB && use_pp(M, K)) {
    // 256-wide tiles, or 224-wide ones when that takes fewer rounds of tiles over the CUs:
    // a 224-wide tile measures about as long as a 256-wide one (its waves' columns straddle
    // weight-scale blocks, one select per promoted fragment), so it only pays when it saves
    // whole rounds.  FP8Q_PP_WIDTH=256|224 forces one.
    const int64_t tm = (M + kBM - 1) / kBM;
    const int64_t t256 = tm * ((N + 255) / 256), t224 = tm * ((N + 223) / 224);
    const int64_t slots = (cus / 8) * 8 > 0 ? (cus / 8) * 8 : cus;
    bool narrow = (t224 + slots - 1) / slots < (t256 + slots - 1) / slots;
    const char *wforce = getenv("FP8Q_PP_WIDTH");
    if (wforce && strcmp(wforce, "256") == 0) narrow = false;
    if (wforce && strcmp(wforce, "224") == 0) narrow = true;
    int64_t tiles = narrow ? t224 : t256;
    if (tiles > 0x7fffffff) return hipErrorInvalidValue;
    // Two-region plan (plan_tile) when the 256 x 256 tiles leave a last round 1/4, 1/2 or
    // 3/4 full: that round's work as one round of 64*hb-row tiles.  FP8Q_PP_PLAN=off keeps
    // the uniform tiles.
    int64_t rb = 0, cb = 0;
    int hb = 0;
    const char *pforce = getenv("FP8Q_PP_PLAN");
    const bool plan_ok = !(pforce && strcmp(pforce, "off") == 0);
    if (plan_ok && !narrow && M % 256 == 0 && N % 256 == 0 && t256 % slots != 0) {
      const int64_t r = t256 % slots;
      for (int h = 3; h >= 1 && hb == 0; --h) {
        if (4 * r != h * slots) continue;
        const int64_t step = h == 3 ? 768 : 256;  // lcm(256, 64h): region A stays 256-row tiled
        for (int64_t R = (M / step) * step; R >= step; R -= step) {
          const int64_t area = slots * 64 * h * 256;  // region B's elements
          if (area % R != 0) continue;
          const int64_t C = area / R;
          if (C % 256 != 0 || C > N) continue;
          rb = R;
          cb = C;
          hb = h;
          break;
        }
      }
      if (hb != 0) tiles = t256 - r + slots;  // q rounds of full tiles and one of region B
    }
    const int64_t grid = hb != 0 ? slots : min(tiles, slots);  // the plan needs one workgroup per slot
    if (narrow)
      hipLaunchKernelGGL(gemm_pp_kernel<7>, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, stream, xq, sa, wq,
                         sb, M, N, K, static_cast<int>(tiles), c, out_f32 ? 1 : 0, int64_t(0), int64_t(0), 0);
    else
      hipLaunchKernelGGL(gemm_pp_kernel<8>, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, stream, xq, sa, wq,
                         sb, M, N, K, static_cast<int>(tiles), c, out_f32 ? 1 : 0, rb, cb, hb);
    return hipGetLastError();
  }
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
  // Each XCD's list holds at most ceil(P/8) groups of every expert (P = tiles_n panels),
  // so slots * ceil(P/8) items; workgroups past an XCD's list exit.
  const int64_t grid = 8 * slots * ((tiles_n + 7) / 8);
  if (grid > 0x7fffffff - 4096 || G > 0x7fffffff) return hipErrorInvalidValue;  // item indices stay in int
  hipLaunchKernelGGL(gemm_grouped_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, stream,
                     xq, sa, wq, sb, offsets, static_cast<int>(G), M_tot, N, K, c, out_f32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace fp8q
