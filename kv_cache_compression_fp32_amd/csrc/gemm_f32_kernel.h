// fp32 matrix-core GEMM kernel template of the compressor's projections
// (gfx950, wave64). Included by gemm_f32.hip, which picks the instances.
//
// C_h[m][n] = sum_k A[m][k] * B_h[n][k] for the two column halves h of the
// output (kv with wkv, score with wgate): "Module compress", Functions,
// linear_f32 (w is [out_dim, in_dim]); "DeepSeek V4.1 . Pool token pairs",
// Compressor listing, forward.
//
// Matrix-core layouts used (lane l of a wavefront):
//   v_mfma_f32_16x16x4_f32: A[l % 16][k-slot l / 16], B[k-slot l / 16][l % 16];
//     accumulator r holds D[4 (l / 16) + r][l % 16].
//   v_mfma_f32_32x32x2_f32: A[l % 32][k-slot l / 32], B[k-slot l / 32][l % 32];
//     accumulator r holds D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
// LDS holds each k tile as [k / 4][row][4] floats (plus one padding row per
// k-group so the 16-byte stores of 8 neighbouring threads hit distinct banks).
// One ds_read_b128 gives a lane 4 consecutive k of its row; MFMA t of a chunk
// takes element t, so k-slot q of MFMA t holds k = chunk_base + 4 q + t for
// both operands and every k is covered once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_launch.h"

namespace kvc {
namespace gemm {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t n) {
  const uint32_t q = n / 8, r = n % 8, x = id % 8, local = id / 8;
  return (x < r) ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

constexpr int kBK = 32;       // k per LDS tile
constexpr int kKG = kBK / 4;  // k-groups of 4 per tile

// MFMA shape traits. KS = k-slots per MFMA (lanes split into KS groups);
// a chunk covers 4 * KS k (one b128 read per fragment, 4 MFMAs).
template <bool BIG> struct Mfma;
template <> struct Mfma<false> {
  static constexpr int D = 16, KS = 4, ACC = 4;
  typedef f4 acc_t;
  __device__ static acc_t run(float a, float b, acc_t c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
  __device__ static int row(int lane, int r) { return 4 * (lane >> 4) + r; }
};
template <> struct Mfma<true> {
  static constexpr int D = 32, KS = 2, ACC = 16;
  typedef f16v acc_t;
  __device__ static acc_t run(float a, float b, acc_t c) { return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0); }
  __device__ static int row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
};

// BM x BN workgroup tile, WM x WN per wavefront, NW wavefronts.
template <int BM, int BN, int WM, int WN, int NW, bool BIG, int MINW>
__global__ __launch_bounds__(NW * 64, MINW) void gemm_f32_kernel(GemmArgs g) {
  using M = Mfma<BIG>;
  constexpr int NT = NW * 64;
  constexpr int WAVES_N = BN / WN;
  static_assert((BM / WM) * (BN / WN) == NW, "wavefront grid must cover the tile");
  constexpr int FM = WM / M::D, FN = WN / M::D;
  constexpr int CH = 4 * M::KS;                  // k per chunk
  constexpr int NCH = kBK / CH;                  // chunks per tile
  constexpr int AL = BM * kKG / NT, BL = BN * kKG / NT;
  static_assert(AL >= 1 && BL >= 1 && BM * kKG % NT == 0 && BN * kKG % NT == 0, "tile/thread mismatch");
  constexpr int AP = BM + 1, BP = BN + 1;
  __shared__ f4 As[2][kKG][AP];
  __shared__ f4 Bs[2][kKG][BP];

  const int64_t m_tiles = (g.m + BM - 1) / BM;
  const int64_t n_tiles = 2 * g.n_half / BN;
  const uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t mt = tile / n_tiles, nt = tile - mt * n_tiles;
  if (mt >= m_tiles) return;
  const int64_t m0 = mt * BM;
  const int64_t n_glob = nt * BN;
  const bool second = n_glob >= g.n_half;
  const int64_t n0 = second ? n_glob - g.n_half : n_glob;
  const float *__restrict__ B = second ? g.b1 : g.b0;
  float *__restrict__ C = (second ? g.c1 : g.c0) + (int64_t)blockIdx.y * g.c_split_stride;
  const int64_t k_len = g.k / g.splits;
  const int64_t k_begin = (int64_t)blockIdx.y * k_len;
  const int kt_count = (int)(k_len / kBK);

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // global -> register prefetch: load u of thread t covers row (t + NT u) / kKG,
  // k-group (t + NT u) % kKG; eight threads read one 128-byte row segment
  const float *a_src[AL];
  const float *b_src[BL];
#pragma unroll
  for (int u = 0; u < AL; ++u) {
    const int li = t + NT * u, r = li / kKG, q = li % kKG;
    int64_t row = m0 + r;
    if (row >= g.m) row = g.m - 1;  // ragged last tile: read a valid row, never store it
    a_src[u] = g.a + row * g.lda + k_begin + 4 * q;
  }
#pragma unroll
  for (int u = 0; u < BL; ++u) {
    const int li = t + NT * u, r = li / kKG, q = li % kKG;
    b_src[u] = B + (n0 + r) * g.ldb + k_begin + 4 * q;
  }
  f4 ra[AL], rb[BL];
  auto gload = [&](int kt) {
#pragma unroll
    for (int u = 0; u < AL; ++u) ra[u] = *reinterpret_cast<const f4 *>(a_src[u] + kt * kBK);
#pragma unroll
    for (int u = 0; u < BL; ++u) rb[u] = *reinterpret_cast<const f4 *>(b_src[u] + kt * kBK);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < AL; ++u) {
      const int li = t + NT * u;
      As[buf][li % kKG][li / kKG] = ra[u];
    }
#pragma unroll
    for (int u = 0; u < BL; ++u) {
      const int li = t + NT * u;
      Bs[buf][li % kKG][li / kKG] = rb[u];
    }
  };

  typename M::acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = typename M::acc_t{};

  const int row_in = lane % M::D, slot = lane / M::D;
  // fragments of two chunks: the next chunk's reads are issued before the
  // current chunk's MFMAs
  f4 fa[2][FM], fb[2][FN];
  auto fload = [&](int buf, int c, int s) {
    const int q = c * M::KS + slot;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[s][i] = As[buf][q][wm * WM + M::D * i + row_in];
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[s][j] = Bs[buf][q][wn * WN + M::D * j + row_in];
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < kt_count; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < kt_count) gload(kt + 1);
    fload(buf, 0, 0);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (c + 1 < NCH) fload(buf, c + 1, (c + 1) & 1);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = M::run(fa[c & 1][i][s], fb[c & 1][j][s], acc[i][j]);
    }
    if (kt + 1 < kt_count) lstore(buf ^ 1);
    __syncthreads();
  }

  const float *bias = second ? g.bias1 : nullptr;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < M::ACC; ++r) {
      const int64_t row = m0 + wm * WM + M::D * i + M::row(lane, r);
      if (row < g.m) {
        float *crow = C + row * g.ldc + n0 + wn * WN + row_in;
        if (bias) {
          const float *brow = bias + ((row % g.bias_seqlen) % g.bias_ratio) * g.ldc + n0 + wn * WN + row_in;
#pragma unroll
          for (int j = 0; j < FN; ++j) crow[M::D * j] = acc[i][j][r] + brow[M::D * j];
        } else {
#pragma unroll
          for (int j = 0; j < FN; ++j) crow[M::D * j] = acc[i][j][r];
        }
      }
    }
}

// Single-LDS-buffer variant with a deeper k tile: BK k per tile (16 k-groups
// at BK = 64), so sixteen neighbouring threads load one 256-byte row segment
// and their 16-byte LDS stores land on 16 distinct bank groups (row pitch of
// BM + 1 k-groups). The next tile is prefetched into registers while the
// current one is multiplied; two barriers per tile (reads done, stores done),
// covered by the second workgroup on the CU. Fragments of the next 16-k chunk
// are read from LDS before the current chunk's MFMAs.
template <int BM, int BN, int WM, int WN, int NW, int BK, int MINW>
__global__ __launch_bounds__(NW * 64, MINW) void gemm_f32_sb_kernel(GemmArgs g) {
  using M = Mfma<false>;
  constexpr int NT = NW * 64;
  constexpr int KG = BK / 4;
  constexpr int WAVES_N = BN / WN;
  static_assert((BM / WM) * (BN / WN) == NW, "wavefront grid must cover the tile");
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int NCH = BK / 16;
  constexpr int AL = BM * KG / NT, BL = BN * KG / NT;
  static_assert(AL >= 1 && BL >= 1 && BM * KG % NT == 0 && BN * KG % NT == 0, "tile/thread mismatch");
  constexpr int AP = BM + 1, BP = BN + 1;
  __shared__ f4 As[KG][AP];
  __shared__ f4 Bs[KG][BP];

  const int64_t m_tiles = (g.m + BM - 1) / BM;
  const int64_t n_tiles = 2 * g.n_half / BN;
  const uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t mt = tile / n_tiles, nt = tile - mt * n_tiles;
  if (mt >= m_tiles) return;
  const int64_t m0 = mt * BM;
  const int64_t n_glob = nt * BN;
  const bool second = n_glob >= g.n_half;
  const int64_t n0 = second ? n_glob - g.n_half : n_glob;
  const float *__restrict__ B = second ? g.b1 : g.b0;
  float *__restrict__ C = (second ? g.c1 : g.c0) + (int64_t)blockIdx.y * g.c_split_stride;
  const int64_t k_len = g.k / g.splits;
  const int64_t k_begin = (int64_t)blockIdx.y * k_len;
  const int kt_count = (int)(k_len / BK);

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const float *a_src[AL];
  const float *b_src[BL];
#pragma unroll
  for (int u = 0; u < AL; ++u) {
    const int li = t + NT * u, r = li / KG, q = li % KG;
    int64_t row = m0 + r;
    if (row >= g.m) row = g.m - 1;  // ragged last tile: read a valid row, never store it
    a_src[u] = g.a + row * g.lda + k_begin + 4 * q;
  }
#pragma unroll
  for (int u = 0; u < BL; ++u) {
    const int li = t + NT * u, r = li / KG, q = li % KG;
    b_src[u] = B + (n0 + r) * g.ldb + k_begin + 4 * q;
  }
  f4 ra[AL], rb[BL];
  auto gload = [&](int kt) {
#pragma unroll
    for (int u = 0; u < AL; ++u) ra[u] = *reinterpret_cast<const f4 *>(a_src[u] + kt * BK);
#pragma unroll
    for (int u = 0; u < BL; ++u) rb[u] = *reinterpret_cast<const f4 *>(b_src[u] + kt * BK);
  };
  auto lstore = [&]() {
#pragma unroll
    for (int u = 0; u < AL; ++u) {
      const int li = t + NT * u;
      As[li % KG][li / KG] = ra[u];
    }
#pragma unroll
    for (int u = 0; u < BL; ++u) {
      const int li = t + NT * u;
      Bs[li % KG][li / KG] = rb[u];
    }
  };

  f4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  const int row_in = lane & 15, slot = lane >> 4;
  f4 fa[2][FM], fb[2][FN];
  auto fload = [&](int c, int sl) {
    const int q = c * 4 + slot;
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[sl][i] = As[q][wm * WM + 16 * i + row_in];
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[sl][j] = Bs[q][wn * WN + 16 * j + row_in];
  };

  gload(0);
  lstore();
  __syncthreads();
  fload(0, 0);
  for (int kt = 0; kt < kt_count; ++kt) {
    if (kt + 1 < kt_count) gload(kt + 1);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (c + 1 < NCH) fload(c + 1, (c + 1) & 1);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = M::run(fa[c & 1][i][s], fb[c & 1][j][s], acc[i][j]);
    }
    __syncthreads();  // every wavefront is done reading this tile
    if (kt + 1 < kt_count) {
      lstore();
      __syncthreads();  // the next tile is in LDS
      fload(0, 0);
    }
  }

  const float *bias = second ? g.bias1 : nullptr;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + wm * WM + 16 * i + M::row(lane, r);
      if (row < g.m) {
        float *crow = C + row * g.ldc + n0 + wn * WN + row_in;
        if (bias) {
          const float *brow = bias + ((row % g.bias_seqlen) % g.bias_ratio) * g.ldc + n0 + wn * WN + row_in;
#pragma unroll
          for (int j = 0; j < FN; ++j) crow[16 * j] = acc[i][j][r] + brow[16 * j];
        } else {
#pragma unroll
          for (int j = 0; j < FN; ++j) crow[16 * j] = acc[i][j][r];
        }
      }
    }
}

template <int BM, int BN, int WM, int WN, int NW, int BK, int MINW>
hipError_t launch_sb(const GemmArgs &g, hipStream_t stream) {
  if (g.n_half % BN != 0 || g.splits < 1 || g.k % (BK * g.splits) != 0 || (g.bias1 && g.splits != 1) ||
      (g.bias1 && (g.bias_seqlen < 1 || g.bias_ratio < 1)))
    return hipErrorInvalidValue;
  const int64_t m_tiles = (g.m + BM - 1) / BM;
  const int64_t n_tiles = 2 * g.n_half / BN;
  hipLaunchKernelGGL((gemm_f32_sb_kernel<BM, BN, WM, WN, NW, BK, MINW>),
                     dim3((uint32_t)(m_tiles * n_tiles), (uint32_t)g.splits), dim3(NW * 64), 0, stream, g);
  return hipGetLastError();
}

// Decode projection (M = batch rows, 64 per row tile in blockIdx.z): 32
// output columns per workgroup (blockIdx.x), the K range split over gridDim.y
// parts and again over the 8 wavefronts of the workgroup. Every A and B value
// is used by one wavefront only, so fragments come straight from global
// memory (lane l reads 4 consecutive k of row l % 16 at k-slot l / 16, the
// layout of v_mfma_f32_16x16x4_f32 with the same k permutation as the tiled
// kernel); the loads of CPW chunks of 16 k are issued before their MFMAs. The
// 8 partial 64 x 32 tiles are summed through LDS in a fixed order.
template <int CPW>
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

  const float *ap[FM];
  const float *bp[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    int64_t row = m0 + 16 * i + row_in;
    if (row >= g.m) row = g.m - 1;  // rows past the batch: read a valid row, never store it
    ap[i] = g.a + row * g.lda + 4 * slot;
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
      for (int i = 0; i < FM; ++i) af[u][i] = *reinterpret_cast<const f4 *>(ap[i] + (c + u) * 16);
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
    for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const f4 *>(ap[i] + c * 16);
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

inline hipError_t launch_decode_gemm(const GemmArgs &g, hipStream_t stream) {
  if (g.n_half % 32 != 0 || g.k % 16 != 0 || g.splits < 1 || g.bias1) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)(2 * g.n_half / 32), (uint32_t)g.splits, (uint32_t)((g.m + 63) / 64));
  hipLaunchKernelGGL(decode_gemm_kernel<4>, grid, dim3(512), 0, stream, g);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int NW, bool BIG, int MINW>
hipError_t launch_tiled(const GemmArgs &g, hipStream_t stream) {
  // every column tile must lie inside one half, every split cover whole k tiles
  if (g.n_half % BN != 0 || g.splits < 1 || g.k % (kBK * g.splits) != 0 || (g.bias1 && g.splits != 1) ||
      (g.bias1 && (g.bias_seqlen < 1 || g.bias_ratio < 1)))
    return hipErrorInvalidValue;
  const int64_t m_tiles = (g.m + BM - 1) / BM;
  const int64_t n_tiles = 2 * g.n_half / BN;
  hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, WM, WN, NW, BIG, MINW>),
                     dim3((uint32_t)(m_tiles * n_tiles), (uint32_t)g.splits), dim3(NW * 64), 0, stream, g);
  return hipGetLastError();
}

}  // namespace gemm
}  // namespace kvc
