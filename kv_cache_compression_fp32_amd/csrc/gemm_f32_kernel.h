// fp32 matrix-core GEMM kernels of the compressor's projections (gfx950,
// wave64). Included by gemm_f32.hip, which picks the instances.
//
// C_h[m][n] = sum_k A[m][k] * B_h[n][k] for the two column halves h of the
// output (kv with wkv, score with wgate): "Module compress", Functions,
// linear_f32 (w is [out_dim, in_dim]); "DeepSeek V4.1 . Pool token pairs",
// Compressor listing, forward.
//
// Matrix-core layout used (lane l of a wavefront), v_mfma_f32_16x16x4_f32:
//   A[l % 16][k-slot l / 16], B[k-slot l / 16][l % 16]; accumulator r holds
//   D[4 (l / 16) + r][l % 16].
// One ds_read_b128 gives a lane 4 consecutive k of its row; MFMA t of a 16-k
// chunk takes element t, so k-slot q of MFMA t holds k = chunk_base + 4 q + t
// for both operands and every k is covered once, in the same order for every
// output element.
//
// Summation order: each output is (p0 + p1) + ..., p_s the chain of MFMAs
// over the k segment [s L, (s + 1) L) of the kKSegments segments
// (kvc_launch.h; the last one to k), L = 32 * floor(k / (32 kKSegments)),
// each chain starting from zero and taking the 16-k chunks in increasing k
// (one chain over all of k when L is 0). The decode projection
// (decode_f32.hip) computes the same chains for one token, so a token's
// projections have the same bits whichever path computes them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.h"
#include "gemm_epilogue.h"
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {
namespace gemm {

constexpr int kBK = 32;  // k per LDS stage

// Prefill projection: BM x BN workgroup tile, WM x WN per wavefront, NW
// wavefronts, two LDS stages of 32 k each. Tiles are loaded with buffer loads
// that write LDS directly (no registers, no LDS store instructions); each load
// instruction of a wavefront fills 1 KiB of LDS: 8 rows of 32 k. LDS holds a
// stage as [rows][32] floats with the 16-byte k-group q of row r at group
// position q ^ (r & 7), so the fragment reads of 8 neighbouring rows hit 8
// distinct bank groups.
// Per tile: the fragments of the first 16-k chunk are read, the second chunk's
// reads are issued behind the first chunk's MFMAs, the next tile's loads go
// out after the tile's last LDS read (to the other stage, which every
// wavefront finished reading before the last barrier), then wait + barrier.
// With DEFER, the tile's last k-slice of MFMAs (operands already in
// registers) runs after the barrier, behind the next tile's first LDS reads.
// Rows of a ragged last row tile are clamped to the last row of A (loaded,
// never stored).
//
// POOL (ratio 4, 256 x 256 tiles of eight 64 x 128 wavefronts): column
// tile nt covers the 64 features 64 nt .. +63, each wavefront's B rows are
// the four 32-row segments of pool_epilogue (gemm_epilogue.h) for its 32
// features, and the tile ends in that pooling epilogue.
template <int BM, int BN, int WM, int WN, int NW, int MINW, bool DEFER, bool POOL = false>
__global__ __launch_bounds__(NW * 64, MINW) void gemm_f32_kernel(GemmArgs g) {
  constexpr int BK = kBK, G = BK / 4;
  constexpr int WAVES_N = BN / WN;
  static_assert((BM / WM) * (BN / WN) == NW, "wavefront grid must cover the tile");
  static_assert(G == 8, "the k-group swizzle assumes 8 groups per row");
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int NCH = BK / 16;
  constexpr int LAST = (NCH - 1) & 1;  // fragment slot of a tile's last chunk
  constexpr int A_INS = BM * BK / 256 / NW, B_INS = BN * BK / 256 / NW;  // 1 KiB loads per wavefront
  static_assert(A_INS >= 1 && B_INS >= 1 && BM * BK % (256 * NW) == 0 && BN * BK % (256 * NW) == 0,
                "tile/wavefront mismatch");
  static_assert(!POOL || (BM == 256 && BN == 256 && WM == 64 && WN == 128 && NW == 8), "pooling tile shape");
  // the stage buffers, reused by the pooling epilogue's branch-B exchange
  constexpr int STAGE_FLOATS = 2 * (BM + BN) * BK;
  constexpr int SMEM_FLOATS = POOL && kPoolXFloats > STAGE_FLOATS ? kPoolXFloats : STAGE_FLOATS;
  __shared__ __attribute__((aligned(16))) float smem[SMEM_FLOATS];
  float(*As)[BM * BK] = reinterpret_cast<float(*)[BM * BK]>(smem);
  float(*Bs)[BN * BK] = reinterpret_cast<float(*)[BN * BK]>(smem + 2 * BM * BK);

  const int64_t m_tiles = (g.m + BM - 1) / BM;
  const int64_t n_tiles = POOL ? g.pool_hd / 64 : 2 * g.n_half / BN;
  const uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t mt = tile / n_tiles, nt = tile - mt * n_tiles;
  if (mt >= m_tiles) return;
  const int64_t m0 = mt * BM;
  const int64_t n_glob = nt * BN;
  const bool second = n_glob >= g.n_half;
  const int64_t n0 = second ? n_glob - g.n_half : n_glob;
  const float *__restrict__ B = second ? g.b1 : g.b0;
  float *__restrict__ C = second ? g.c1 : g.c0;
  const int kt_count = (int)(g.k / BK);

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // Load u of this wavefront fills LDS bytes [1 KiB (wave INS + u), +1 KiB):
  // lane l -> row 8 (wave INS + u) + l / 8, group position l % 8, which holds
  // k-group lq = (l % 8) ^ ((l / 8) & 7). Buffer resources start at the
  // tile's first row; the k offset is wavefront-uniform.
  const int64_t a_rows = (g.m - m0 < BM) ? (g.m - m0) : BM;
  const i32x4 a_rsrc = make_rsrc(g.a + m0 * g.lda, (uint32_t)(a_rows * g.lda * 4));
  // B rows of this wavefront's loads: n0 + 8 (wave INS + u) + l / 8; with
  // POOL, the 32 rows of segment wave % 4 for features f0 + 32 (wave / 4) ..
  // (the wavefront's own resource, its rows from the resource's start)
  const int64_t f0 = 64 * nt;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const i32x4 b_rsrc =
      POOL ? make_rsrc((wave_u & 3) < 2 ? g.b0 + (((wave_u & 1) * g.pool_hd + f0 + 32 * (wave_u >> 2)) * g.ldb)
                                        : g.b1 + (((wave_u & 1) * g.pool_hd + f0 + 32 * (wave_u >> 2)) * g.ldb),
                       (uint32_t)(32 * g.ldb * 4))
           : make_rsrc(B + n0 * g.ldb, (uint32_t)(BN * g.ldb * 4));
  const int lr = lane / G, lq = (lane % G) ^ (lr & 7);
  uint32_t a_voff[A_INS];
#pragma unroll
  for (int u = 0; u < A_INS; ++u) {
    int64_t r = 8 * (wave * A_INS + u) + lr;
    if (r >= a_rows) r = a_rows - 1;  // ragged last tile: read a valid row, never store it
    a_voff[u] = (uint32_t)((r * g.lda + 4 * lq) * 4);
  }
  const uint32_t b_voff = (uint32_t)(((POOL ? 0 : 8 * wave * B_INS) + lr) * g.ldb * 4 + 4 * lq * 4);
  auto issue = [&](int kt, int st) {
    const uint32_t koff = (uint32_t)(kt * BK * 4);
#pragma unroll
    for (int u = 0; u < A_INS; ++u)
      buffer_load_lds(a_rsrc, (lds_u32 *)(&As[st][256 * (wave * A_INS + u)]), 16, (int32_t)a_voff[u],
                      (int32_t)koff, 0, 0);
#pragma unroll
    for (int u = 0; u < B_INS; ++u)
      buffer_load_lds(b_rsrc, (lds_u32 *)(&Bs[st][256 * (wave * B_INS + u)]), 16, (int32_t)b_voff,
                      (int32_t)(koff + (uint32_t)(8 * u * g.ldb * 4)), 0, 0);
  };

  f4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  const int row_in = lane & 15, slot = lane >> 4;
  f4 fa[2][FM], fb[2][FN];
  auto fload = [&](int st, int c, int sl) {
    const int q = c * 4 + slot;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WM + 16 * i + row_in;
      fa[sl][i] = *reinterpret_cast<const f4 *>(&As[st][r * BK + 4 * (q ^ (r & 7))]);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = wn * WN + 16 * j + row_in;
      fb[sl][j] = *reinterpret_cast<const f4 *>(&Bs[st][r * BK + 4 * (q ^ (r & 7))]);
    }
  };
  auto mfma_slice = [&](int sl, int s) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[sl][i][s], fb[sl][j][s], acc[i][j], 0, 0, 0);
  };

  // The k segments (see the header): stages [0, L), [L, 2 L), .. of 32 k, L
  // = floor(k / (32 kKSegments)), the last segment to k / 32; each segment's
  // chain starts from zero, and the running sum p0, then p0 + p1, ..
  // waits between segments in the tile's own output positions of C, which no
  // other tile reads or writes (a ragged last row tile, whose rows past the
  // end of A do not exist in C, uses g.rag instead: BM rows of its column
  // tile's BN columns). The sum is kept lane-major, each store or load
  // instruction of a wavefront covering one contiguous KiB: wavefront w owns
  // rows 32 w .. 32 w + 31 of the tile, and its accumulator fragment q (of
  // FM x FN) goes to row 32 w + q (BN = 256; with BN = 128, rows 32 w + 2 q
  // and 32 w + 2 q + 1), lane l at 16-byte position l of that KiB (with POOL
  // the four 256-byte pieces of the row's kv branch A, kv branch B, score
  // branch A and score branch B columns of the tile's 64 features). The
  // lane's pointer is derived from a fresh lane id where it is used, so that
  // nothing extra stays live through the k loop.
  const int kt_seg = (int)(g.k / (32 * kKSegments));
  constexpr int NQ = FM * FN;  // accumulator fragments per lane
  static_assert(BM / NW == 32 && (BN == 256 || BN == 128) && NQ * 64 * 16 == 32 * BN * 4,
                "the lane-major layout covers the wavefront's 32 rows of the tile");
  constexpr int QROWS = BN == 256 ? 1 : 2;  // tile rows between fragment slots q and q + 1
  auto sum_ptr = [&](int64_t &stride) -> float * {
    const int l = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int64_t r0 = 32 * wave_u + (BN == 256 ? 0 : (l >> 5));  // the lane's row for q = 0
    const int c4 = BN == 256 ? 4 * l : 4 * (l & 31);                // the lane's column offset in a row
    if (m0 + BM > g.m) {
      stride = BN;
      return g.rag + nt * BM * BN + r0 * BN + c4;
    }
    stride = g.ldc;
    if constexpr (POOL) {
      const int piece = l >> 4;
      return (piece >= 2 ? g.c1 : g.c0) + (m0 + r0) * g.ldc + (piece & 1) * g.pool_hd + f0 + 4 * (l & 15);
    } else {
      return C + (m0 + r0) * g.ldc + n0 + c4;
    }
  };
  // mode 0: store the accumulators; 1: add them to the stored sum and store
  // that; 2: add them to the stored sum (the final sum). The accumulators
  // restart from zero after modes 0 and 1. Loads go in chunks (8 fragments
  // inside the k loop, 16 after it), each drained before the next, so that
  // few registers are held.
  auto spill = [&](auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
    int64_t stride;
    float *p = sum_ptr(stride);
    if constexpr (MODE == 0) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) *reinterpret_cast<f4 *>(p + QROWS * q * stride) = acc[q / FN][q % FN];
    } else {
      constexpr int CH = MODE == 2 ? (NQ < 16 ? NQ : 16) : (NQ < 8 ? NQ : 8);
#pragma unroll
      for (int q0 = 0; q0 < NQ; q0 += CH) {
        f4 t[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) t[u] = *reinterpret_cast<const f4 *>(p + QROWS * (q0 + u) * stride);
#pragma unroll
        for (int u = 0; u < CH; ++u) {
          f4 &a = acc[(q0 + u) / FN][(q0 + u) % FN];
          const f4 sum = f4{t[u][0] + a[0], t[u][1] + a[1], t[u][2] + a[2], t[u][3] + a[3]};
          if constexpr (MODE == 1) *reinterpret_cast<f4 *>(p + QROWS * (q0 + u) * stride) = sum;
          else a = sum;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (MODE != 2) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
    }
  };

  issue(0, 0);
  wait_vm0();
  __syncthreads();
#pragma clang loop unroll(disable)
  for (int kt = 0; kt < kt_count; ++kt) {
    const int st = kt & 1;
    fload(st, 0, 0);
    if (DEFER && kt > 0) {
      __builtin_amdgcn_sched_barrier(0);
      mfma_slice(LAST, 3);
      __builtin_amdgcn_sched_barrier(0);
    }
    // a segment ended with the previous stage: p0 is stored, later ones join
    // the stored sum (the previous stage's fragment registers are free here)
    if (kKSegments > 1 && kt_seg > 0 && kt <= (kKSegments - 1) * kt_seg && kt % kt_seg == 0 && kt > 0) {
      if (kKSegments == 2 || kt == kt_seg) spill(std::integral_constant<int, 0>{});
      else spill(std::integral_constant<int, 1>{});
    }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (c + 1 < NCH) fload(st, c + 1, (c + 1) & 1);
      // unconditional, so the loop body stays one block: the last iteration
      // reloads its own tile into the idle stage, which is never read
      if (c == NCH - 1) issue(kt + 1 < kt_count ? kt + 1 : kt, st ^ 1);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (!(DEFER && c == NCH - 1 && s == 3)) mfma_slice(c & 1, s);
    }
    __builtin_amdgcn_sched_barrier(0);  // the tile's MFMAs stay ahead of the wait
    wait_vm0();                         // this wavefront's loads of the next tile landed
    __syncthreads();                    // everyone's landed; everyone is done reading this stage
  }
  if (DEFER) mfma_slice(LAST, 3);
  // (p0 + p1) + .. (each lane reads back what it stored); the outputs then
  // go to positions whose stored sums other lanes read, so every wavefront
  // first finishes its reads
  if (kKSegments > 1 && kt_seg > 0) {
    spill(std::integral_constant<int, 2>{});
    __syncthreads();
  }

  if constexpr (POOL) {
    pool_epilogue<WM, WN>(g, acc, smem, m0, f0, wm, wn, lane);
  } else {
    store_tile<FM, FN>(g, acc, C, second ? g.bias1 : nullptr, m0 + wm * WM, n0 + wn * WN, lane);
  }
}

__device__ __forceinline__ f4 load_a4(const float *p) { return *reinterpret_cast<const f4 *>(p); }
// 4 bf16 values promoted to f32 (exact)
__device__ __forceinline__ f4 load_a4(const uint16_t *p) {
  const uint2 v = *reinterpret_cast<const uint2 *>(p);
  return f4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
            __uint_as_float(v.y & 0xffff0000u)};
}

// Decode projection (M = batch rows, 64 per row tile in blockIdx.z): 32
// output columns per workgroup (blockIdx.x), the K range split over gridDim.y
// parts and again over the 8 wavefronts of the workgroup. Every A and B value
// is used by one wavefront only, so fragments come straight from global
// memory (lane l reads 4 consecutive k of row l % 16 at k-slot l / 16, the
// layout of v_mfma_f32_16x16x4_f32 with the same k permutation as the tiled
// kernel); the loads of CPW chunks of 16 k are issued before their MFMAs. The
// 8 partial 64 x 32 tiles are summed through LDS in a fixed order. Used for
// bf16 x rows (TA = uint16_t, promoted on load); f32 rows take the decode
// kernel of decode_f32.hip, which sums as the prefill does.
template <int CPW, typename TA>
__global__ __launch_bounds__(512, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_gemm_kernel(GemmArgs g) {
  constexpr int NWV = 8, FM = 4, FN = 2;
  __shared__ float red[NWV][64][33];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n_glob = (int64_t)blockIdx.x * 32;
  const bool second = n_glob >= g.n_half;
  const int64_t n0 = second ? n_glob - g.n_half : n_glob;
  const float *__restrict__ B = second ? g.b1 : g.b0;
  float *__restrict__ C = (second ? g.c1 : g.c0) + (int64_t)blockIdx.y * g.c_split_stride;
  const int64_t m0 = (int64_t)blockIdx.z * 64;
  const int64_t chunks = g.k / 16;
  const int64_t parts = (int64_t)gridDim.y * NWV;
  const int64_t me = (int64_t)blockIdx.y * NWV + wave;
  const int64_t c_begin = chunks * me / parts, c_end = chunks * (me + 1) / parts;
  const int row_in = lane & 15, slot = lane >> 4;

  const TA *A;
  if constexpr (sizeof(TA) == 2) A = g.a16; else A = g.a;
  const TA *ap[FM];
  const float *bp[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    int64_t row = m0 + 16 * i + row_in;
    if (row >= g.m) row = g.m - 1;  // rows past the batch: read a valid row, never store it
    ap[i] = A + row * g.lda + 4 * slot;
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) bp[j] = B + (n0 + 16 * j + row_in) * g.ldb + 4 * slot;

  f4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  int64_t c = c_begin;
  for (; c + CPW <= c_end; c += CPW) {
    f4 af[CPW][FM], bf[CPW][FN];
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
#pragma unroll
      for (int i = 0; i < FM; ++i) af[u][i] = load_a4(ap[i] + (c + u) * 16);
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[u][j] = *reinterpret_cast<const f4 *>(bp[j] + (c + u) * 16);
    }
    // keep every load of the group ahead of the MFMAs (all in flight at once)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < CPW; ++u)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[u][i][s], bf[u][j][s], acc[i][j], 0, 0, 0);
  }
  for (; c < c_end; ++c) {
    f4 af[FM], bf[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = load_a4(ap[i] + c * 16);
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[j] = *reinterpret_cast<const f4 *>(bp[j] + c * 16);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][s], bf[j][s], acc[i][j], 0, 0, 0);
  }

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][16 * i + 4 * slot + r][16 * j + row_in] = acc[i][j][r];
  __syncthreads();
  const int row = threadIdx.x >> 3, col = 4 * (threadIdx.x & 7);
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    sum.x += red[w][row][col];
    sum.y += red[w][row][col + 1];
    sum.z += red[w][row][col + 2];
    sum.w += red[w][row][col + 3];
  }
  if (m0 + row < g.m) *reinterpret_cast<float4 *>(C + (m0 + row) * g.ldc + n0 + col) = sum;
}

// Decode projection of bf16 rows (the split-K partials of launch_gemm's
// kDecode shape); f32 rows take decode_f32.hip's kernel instead.
inline hipError_t launch_decode_gemm(const GemmArgs &g, hipStream_t stream) {
  if (!g.a16 || g.n_half % 32 != 0 || g.k % 16 != 0 || g.splits < 1 || g.bias1) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)(2 * g.n_half / 32), (uint32_t)g.splits, (uint32_t)((g.m + 63) / 64));
  hipLaunchKernelGGL((decode_gemm_kernel<4, uint16_t>), grid, dim3(512), 0, stream, g);
  return hipGetLastError();
}

inline hipError_t launch_pooling(const GemmArgs &g, hipStream_t stream) {
  // whole 32-k stages, 64-feature column tiles, 4-token blocks aligned with
  // the flattened rows, tile rows addressable with 32-bit buffer offsets
  if (g.k % kBK != 0 || g.pool_hd % 64 != 0 || g.ldc != 2 * g.pool_hd || g.lda < g.k || g.ldb < g.k ||
      g.m != g.pool_batch * g.pool_seqlen || (g.pool_batch > 1 && g.pool_seqlen % 4 != 0) || !g.pooled ||
      (g.m % 256 != 0 && !g.rag) ||
      (int64_t)256 * g.lda * 4 > INT32_MAX || (int64_t)32 * g.ldb * 4 > INT32_MAX)
    return hipErrorInvalidValue;
  const int64_t m_tiles = (g.m + 255) / 256;
  hipLaunchKernelGGL((gemm_f32_kernel<256, 256, 64, 128, 8, 1, true, true>),
                     dim3((uint32_t)(m_tiles * (g.pool_hd / 64))), dim3(512), 0, stream, g);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int NW, int MINW, bool DEFER>
hipError_t launch_tiled(const GemmArgs &g, hipStream_t stream) {
  // every column tile inside one half, whole k tiles, and a tile's rows
  // addressable by a 32-bit buffer offset
  if (g.n_half % BN != 0 || g.splits != 1 || g.k % kBK != 0 || (g.m % BM != 0 && !g.rag) ||
      (g.bias1 && (g.bias_seqlen < 1 || g.bias_ratio < 1 || (g.bias_ratio & (g.bias_ratio - 1)) != 0)) || g.lda < g.k || g.ldb < g.k ||
      (int64_t)BM * g.lda * 4 > INT32_MAX || (int64_t)BN * g.ldb * 4 > INT32_MAX)
    return hipErrorInvalidValue;
  const int64_t m_tiles = (g.m + BM - 1) / BM;
  const int64_t n_tiles = 2 * g.n_half / BN;
  hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, WM, WN, NW, MINW, DEFER>),
                     dim3((uint32_t)(m_tiles * n_tiles)), dim3(NW * 64), 0, stream, g);
  return hipGetLastError();
}

}  // namespace gemm
}  // namespace kvc
