// fp32 projection GEMM of the compressor on gfx950 matrix cores.
//
// kv = x . wkv^T and score = x . wgate^T with f32 operands and f32 results
// ("Module compress", Functions, linear_f32: w is [out_dim, in_dim];
// "DeepSeek V4.1 . Pool token pairs", Compressor listing, forward). Both
// operands are K-contiguous, so one kernel computes C_h = A . B_h^T for the two
// weight matrices, choosing the half by the workgroup's column tile.
//
// Design (CDNA4, wave64):
//   - v_mfma_f32_16x16x4_f32: lane l supplies A[i = l % 16][k] and
//     B[k][j = l % 16] for k-slot l / 16, and receives D[4 (l / 16) + r][l % 16]
//     in accumulator r.
//   - Tiles of 32 k are staged in LDS as [k/4][row][4] floats (one padding row
//     per k-group keeps the 16-byte stores conflict-free), so that one
//     ds_read_b128 gives a lane the 4 consecutive k of its row. The four
//     MFMAs of a 16-k chunk take element t of that vector: in MFMA t, k-slot q
//     holds k = 16 kk + 4 q + t for both operands, which covers every k once.
//   - 256 threads = 4 wavefronts per workgroup, each owning a WM x WN sub-tile
//     of FM x FN 16x16 blocks; LDS is double-buffered with a register
//     prefetch of the next k tile, one barrier per k tile.
//   - Workgroups are remapped so each XCD walks a contiguous range of output
//     tiles, column tiles fastest, so an A row tile is reused from that XCD's
//     L2 by all column tiles.
//   - K can be split over gridDim.y (decode, where M is the batch) with each
//     split writing its own partial sums.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_launch.h"

namespace kvc {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t n) {
  const uint32_t q = n / 8, r = n % 8, x = id % 8, local = id / 8;
  return (x < r) ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

constexpr int kBK = 32;        // k per LDS tile
constexpr int kKG = kBK / 4;   // k-groups of 4 per tile

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256, 2) void gemm_f32_kernel(GemmArgs g) {
  constexpr int WAVES_N = BN / WN;
  static_assert((BM / WM) * (BN / WN) == 4, "four wavefronts per workgroup");
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int AL = BM * kKG / 256, BL = BN * kKG / 256;  // float4 loads per thread
  static_assert(AL >= 1 && BL >= 1, "tile too small for 256 threads");
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

  // global -> register prefetch coordinates: load u of thread t covers row
  // (t + 256u) / kKG, k-group (t + 256u) % kKG; eight threads read one 128-byte
  // row segment
  const float *a_src[AL];
  const float *b_src[BL];
#pragma unroll
  for (int u = 0; u < AL; ++u) {
    const int li = t + 256 * u, r = li / kKG, q = li % kKG;
    int64_t row = m0 + r;
    if (row >= g.m) row = g.m - 1;  // ragged last tile: read a valid row, never store it
    a_src[u] = g.a + row * g.lda + k_begin + 4 * q;
  }
#pragma unroll
  for (int u = 0; u < BL; ++u) {
    const int li = t + 256 * u, r = li / kKG, q = li % kKG;
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
      const int li = t + 256 * u;
      As[buf][li % kKG][li / kKG] = ra[u];
    }
#pragma unroll
    for (int u = 0; u < BL; ++u) {
      const int li = t + 256 * u;
      Bs[buf][li % kKG][li / kKG] = rb[u];
    }
  };

  f4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  const int row_in = lane & 15, slot = lane >> 4;
  for (int kt = 0; kt < kt_count; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < kt_count) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      f4 af[FM], bf[FN];
      const int q = kk * 4 + slot;
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = As[buf][q][wm * WM + 16 * i + row_in];
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[j] = Bs[buf][q][wn * WN + 16 * j + row_in];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][s], bf[j][s], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < kt_count) lstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + wm * WM + 16 * i + 4 * slot + r;
      if (row < g.m) {
#pragma unroll
        for (int j = 0; j < FN; ++j) C[row * g.ldc + n0 + wn * WN + 16 * j + row_in] = acc[i][j][r];
      }
    }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_tiled(const GemmArgs &g, hipStream_t stream) {
  const int64_t m_tiles = (g.m + BM - 1) / BM;
  const int64_t n_tiles = 2 * g.n_half / BN;
  hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, WM, WN>), dim3((uint32_t)(m_tiles * n_tiles), (uint32_t)g.splits),
                     dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace

int gemm_tile_m(GemmShape s) { return s == GemmShape::kPrefill ? 128 : 64; }
int gemm_tile_n(GemmShape s) { return s == GemmShape::kPrefill ? 128 : 64; }

hipError_t launch_gemm(const GemmArgs &g, GemmShape shape, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  if (shape == GemmShape::kPrefill) return launch_tiled<128, 128, 64, 64>(g, stream);
  return launch_tiled<64, 64, 32, 32>(g, stream);
}

}  // namespace kvc
