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
// into the FP32 accumulator with one FMA per element, acc = P * (sa*sb) + acc.  That FMA
// runs on the vector ALU while the matrix core works on the next MFMA.
//
// Workgroup tile 256(M) x 256(N), K step 128 (= the scale block), 8 waves in a 4(M) x 2(N)
// grid, each owning 64 x 128 outputs (128 FP32 accumulator VGPRs).  The MFMA takes the
// weight fragment as its A operand and the activation fragment as B, so every lane owns
// one output row m and four consecutive columns n: one activation scale per fragment row
// and 8- or 16-byte output stores.
//
// Operand staging: both 256x128-byte stages live in LDS, double buffered (4 x 32 KB).
// gfx950's global_load_lds_dwordx4 moves 16 B per lane straight from global memory into
// LDS; each wave's load fills 1 KB = 8 rows.  The lane->address map applies an XOR swizzle
// of the 16-byte chunk index with the row (row & 7) so that the fragment reads
// (ds_read_b128, 16 rows of one chunk column) hit distinct banks.  The two buffers are
// separate LDS arrays, so the compiler can see that reading one does not wait for the
// loads in flight into the other.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q_launch.h"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
#define FP8Q_LDS __attribute__((address_space(3)))

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 128;
constexpr int kThreads = 512;
constexpr int kStage = kBM * kBK;  // bytes of one operand stage (kBM == kBN)
constexpr int kGroupM = 8;         // M tiles per raster group (L2 reuse of weight panels)

__device__ __forceinline__ int swz(int row) { return row & 7; }

// Buffer resource (gfx9 family layout) over `bytes` bytes at `p`; loads at or past the
// end return zeros, which is how rows beyond the tile's valid range are filled.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// Per-lane byte offsets of the four 16-byte pieces a lane moves for one 256-row x 128-byte
// stage: wave w fills LDS chunks c = 8*i + w (8 rows each, 1 KB); lane p of chunk c lands
// at LDS row 8c + p/8, slot p%8, and fetches global chunk slot ^ swz(row) of that row.
// The same offsets serve both operands (both tiles are 256 rows with row stride K).
__device__ __forceinline__ void stage_offsets(int64_t K, int wave, int lane, uint32_t off[4]) {
  const int r_in = lane >> 3;
  const int slot = lane & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (8 * i + wave) + r_in;
    off[i] = static_cast<uint32_t>(row) * static_cast<uint32_t>(K) + static_cast<uint32_t>((slot ^ swz(row)) << 4);
  }
}

// Copy one stage (K bytes [koff, koff + 128) of all 256 tile rows) into LDS.
__device__ __forceinline__ void stage_load(__amdgpu_buffer_rsrc_t rsrc, const uint32_t off[4], uint32_t koff,
                                           FP8Q_LDS uint8_t *lds, int wave) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FP8Q_LDS void *)(lds + (8 * i + wave) * 1024), 16,
                                             static_cast<int>(off[i]), static_cast<int>(koff), 0, 0);
}

// One MFMA operand fragment: row `row` of the stage, K bytes [32*kg, 32*kg + 32).
__device__ __forceinline__ v8i frag(const FP8Q_LDS uint8_t *lds, int row, int kg) {
  const FP8Q_LDS uint8_t *rp = lds + row * kBK;
  const v4i lo = *reinterpret_cast<const FP8Q_LDS v4i *>(rp + (((2 * kg) ^ swz(row)) << 4));
  const v4i hi = *reinterpret_cast<const FP8Q_LDS v4i *>(rp + (((2 * kg + 1) ^ swz(row)) << 4));
  return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
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
  const uint8_t *w; // weight matrix of the tile's expert, [N][K]
  const float *sb;  // its block scales, [N/128][K/128]
};

__device__ __forceinline__ bool dense_tile(int64_t M, int64_t N, const uint8_t *wq, const float *sb,
                                           Tile &t) {
  const int tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  const int tiles_n = static_cast<int>((N + kBN - 1) / kBN);
  const int total = tiles_m * tiles_n;
  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous run of
  // logical tiles (a bijection on [0, total)) so that its L2 sees neighbouring tiles.
  const int bid = blockIdx.x;
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
  t.n0 = static_cast<int64_t>(tn) * kBN;
  t.w = wq;
  t.sb = sb;
  return true;
}

// Grouped: blockIdx.y is the N tile, blockIdx.x enumerates the M tiles of all experts in
// order (expert g contributes ceil(n_g / 256) tiles).  Offsets come from device memory;
// every range is clamped to [0, M_tot).
__device__ __forceinline__ bool grouped_tile(const int32_t *__restrict__ offsets, int G, int64_t M_tot,
                                             int64_t N, int64_t K, const uint8_t *wq, const float *sb,
                                             Tile &t) {
  const int slot = blockIdx.x;
  int cum = 0;
  int64_t lo = 0;
  for (int g = 0; g < G; ++g) {
    int64_t a = offsets[g], b = offsets[g + 1];
    a = a < 0 ? 0 : (a > M_tot ? M_tot : a);
    b = b < a ? a : (b > M_tot ? M_tot : b);
    const int tiles = static_cast<int>((b - a + kBM - 1) / kBM);
    if (slot < cum + tiles) {
      lo = a + static_cast<int64_t>(slot - cum) * kBM;
      t.m_begin = lo;
      t.rows = static_cast<int>(min(static_cast<int64_t>(kBM), b - lo));
      t.n0 = static_cast<int64_t>(blockIdx.y) * kBN;
      t.w = wq + static_cast<int64_t>(g) * N * K;
      t.sb = sb + static_cast<int64_t>(g) * (N / 128) * (K / 128);
      return true;
    }
    cum += tiles;
  }
  return false;
}

template <bool kGrouped>
__global__ __launch_bounds__(kThreads, 1) void gemm_blockscaled_kernel(
    const uint8_t *__restrict__ xq, const float *__restrict__ sa, const uint8_t *__restrict__ wq,
    const float *__restrict__ sb, const int32_t *__restrict__ offsets, int G, int64_t M, int64_t N,
    int64_t K, void *__restrict__ c, int out_f32) {
  __shared__ __attribute__((aligned(1024))) uint8_t sx0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sw0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sx1[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sw1[kStage];

  Tile t;
  if (kGrouped) {
    if (!grouped_tile(offsets, G, M, N, K, wq, sb, t)) return;
  } else {
    dense_tile(M, N, wq, sb, t);
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1;  // 0..3: rows wm*64 .. +63
  const int wn = wave & 1;   // 0..1: cols wn*128 .. +127
  const int KB = static_cast<int>(K >> 7);
  const int NB = static_cast<int>(N >> 7);
  const int l16 = lane & 15;
  const int kg = lane >> 4;

  // Operand tiles as buffer resources: rows past the valid range read as zeros.
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(xq + t.m_begin * K, static_cast<uint32_t>(t.rows * K));
  const int rows_w = static_cast<int>(min(static_cast<int64_t>(kBN), N - t.n0));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(t.w + t.n0 * K, static_cast<uint32_t>(rows_w * K));
  uint32_t off[4];
  stage_offsets(K, wave, lane, off);

  // activation-scale rows of this lane (one per 16-row fragment), clamped into the tile
  int srow[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int r = wm * 64 + f * 16 + l16;
    srow[f] = static_cast<int>(t.m_begin) + (r < t.rows ? r : t.rows - 1);
  }
  int nb = static_cast<int>((t.n0 + wn * 128) >> 7);  // this wave's 128-column block
  if (nb > NB - 1) nb = NB - 1;
  const float *sbrow = t.sb + static_cast<int64_t>(nb) * KB;

  v4f acc[4][8];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[f][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  float sa_cur[4], sa_nxt[4];
  float sb_cur, sb_nxt = 0.0f;

  FP8Q_LDS uint8_t *lx0 = (FP8Q_LDS uint8_t *)sx0;
  FP8Q_LDS uint8_t *lw0 = (FP8Q_LDS uint8_t *)sw0;
  FP8Q_LDS uint8_t *lx1 = (FP8Q_LDS uint8_t *)sx1;
  FP8Q_LDS uint8_t *lw1 = (FP8Q_LDS uint8_t *)sw1;
  stage_load(rx, off, 0, lx0, wave);
  stage_load(rw, off, 0, lw0, wave);
#pragma unroll
  for (int f = 0; f < 4; ++f) sa_cur[f] = sa[srow[f]];
  sb_cur = sbrow[0];
#pragma unroll
  for (int f = 0; f < 4; ++f) sa_nxt[f] = 0.0f;

  // One K block: wait for its stage, start the copy of the next one into the other
  // buffer, then 32 MFMAs (one per 16x16 fragment pair) each folded into the FP32
  // accumulator with its scale.  The body is branch-free (at the last block the copy just
  // repeats that block), so the promotion FMAs stay next to their MFMAs.
  auto step = [&](const FP8Q_LDS uint8_t *cx, const FP8Q_LDS uint8_t *cw, FP8Q_LDS uint8_t *nx,
                  FP8Q_LDS uint8_t *nw, int kb) {
    // Stage kb has landed in LDS once every wave's own copies are done (vmcnt(0) before
    // the barrier: the compiler's fence does not count direct-to-LDS loads), and after
    // the barrier every wave is also done reading the other buffer.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int kn = kb + 1 < KB ? kb + 1 : kb;
    const uint32_t koff = static_cast<uint32_t>(kn) * kBK;
    stage_load(rx, off, koff, nx, wave);
    stage_load(rw, off, koff, nw, wave);
    const float *sak = sa + static_cast<int64_t>(kn) * M;
#pragma unroll
    for (int f = 0; f < 4; ++f) sa_nxt[f] = sak[srow[f]];
    sb_nxt = sbrow[kn];
    float scl[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) scl[f] = sa_cur[f] * sb_cur;
    v8i xf[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) xf[f] = frag(cx, wm * 64 + f * 16 + l16, kg);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const v8i wf = frag(cw, wn * 128 + j * 16 + l16, kg);
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const v4f p = mfma_block(wf, xf[f]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[f][j][i] = __builtin_fmaf(p[i], scl[f], acc[f][j][i]);
        asm volatile("" : "+v"(acc[f][j]));  // keep the promotion here, not sunk later
      }
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) sa_cur[f] = sa_nxt[f];
    sb_cur = sb_nxt;
  };

  int kb = 0;
  for (; kb + 1 < KB; kb += 2) {
    step(lx0, lw0, lx1, lw1, kb);
    step(lx1, lw1, lx0, lw0, kb + 1);
  }
  if (kb < KB) step(lx0, lw0, lx1, lw1, kb);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the last (repeated) copy

  // Epilogue: lane owns row m = m_begin + wm*64 + f*16 + l16 and columns
  // n0 + wn*128 + j*16 + 4*kg + {0..3}.
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int r = wm * 64 + f * 16 + l16;
    if (r >= t.rows) continue;
    const int64_t m = t.m_begin + r;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t n = t.n0 + wn * 128 + j * 16 + 4 * kg;
      if (n >= N) continue;
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

hipError_t launch_gemm(const uint8_t *xq, const float *sa, const uint8_t *wq, const float *sb,
                       int64_t M, int64_t N, int64_t K, void *c, bool out_f32, hipStream_t stream) {
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_blockscaled_kernel<false>, dim3(static_cast<uint32_t>(tiles)), dim3(kThreads),
                     0, stream, xq, sa, wq, sb, static_cast<const int32_t *>(nullptr), 1, M, N, K, c,
                     out_f32 ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const uint8_t *xq, const float *sa, const uint8_t *wq, const float *sb,
                               const int32_t *offsets, int64_t G, int64_t M_tot, int64_t N, int64_t K,
                               void *c, bool out_f32, hipStream_t stream) {
  // Upper bound on sum_g ceil(n_g / 256) without reading the offsets on the host.
  const int64_t slots = (M_tot + kBM - 1) / kBM + G;
  const int64_t tiles_n = (N + kBN - 1) / kBN;
  if (slots > 0x7fffffff || tiles_n > 65535 || G > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_blockscaled_kernel<true>, dim3(static_cast<uint32_t>(slots), static_cast<uint32_t>(tiles_n)),
                     dim3(kThreads), 0, stream, xq, sa, wq, sb, offsets, static_cast<int>(G), M_tot, N, K,
                     c, out_f32 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace fp8q
