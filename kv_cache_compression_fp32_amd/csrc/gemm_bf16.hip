// bf16 matrix-core GEMM of the ratio-1 compressor's projection (gfx950,
// wave64): C[m][n] = sum_k A[m][k] * B[n][k] with bf16 A (hidden states) and
// B (wkv, [head_dim, dim]), f32 accumulation and f32 output. "DeepSeek V4.1 .
// Pool token pairs", Compressor listing (__init__: wkv stays in the
// checkpoint's bf16 at ratio 1; forward: the ratio-1 branch); "Module
// compress", CompressorWeights.
//
// Matrix-core layout (lane l), v_mfma_f32_16x16x32_bf16: lane l supplies 8
// consecutive k of row l % 16 of A and of column l % 16 of B, k-group l / 16
// of the 32; accumulator r holds D[4 (l / 16) + r][l % 16]. A and B use the
// same lane -> k mapping, so every product pairs matching k.
//
// Structure as the fp32 projection kernel: two LDS stages of 64 k, filled by
// buffer loads that write LDS directly (one instruction per 8 rows x 64 k =
// 1 KiB), rows of 128 bytes holding 8 k-groups of 8 bf16 with group q of row r
// at position q ^ (r & 7); each stage is two 32-k chunks, the second chunk's
// fragments read behind the first chunk's MFMAs, the next stage's loads issued
// after the stage's last LDS read. With DEFER the second chunk's MFMAs run
// after the barrier, behind the next stage's first fragment reads.
#include "gemm_common.h"
#include "kvc_launch.h"

namespace kvc {
namespace gemm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kBKH = 64;  // k (bf16 elements) per LDS stage

template <int BM, int BN, int WM, int WN, int NW, int MINW, bool DEFER>
__global__ __launch_bounds__(NW * 64, MINW) void gemm_bf16_kernel(GemmBf16Args g) {
  constexpr int BK = kBKH, G = 8;  // 8 groups of 8 bf16 per 128-byte row
  constexpr int WAVES_N = BN / WN;
  static_assert((BM / WM) * (BN / WN) == NW, "wavefront grid must cover the tile");
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int A_INS = BM * BK / 512 / NW, B_INS = BN * BK / 512 / NW;  // 1 KiB loads per wavefront
  static_assert(A_INS >= 1 && B_INS >= 1 && BM * BK % (512 * NW) == 0 && BN * BK % (512 * NW) == 0,
                "tile/wavefront mismatch");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];

  const int64_t m_tiles = (g.m + BM - 1) / BM;
  const int64_t n_tiles = g.n / BN;
  const uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t mt = tile / n_tiles, nt = tile - mt * n_tiles;
  if (mt >= m_tiles) return;
  const int64_t m0 = mt * BM, n0 = nt * BN;
  const int kt_count = (int)(g.k / BK);

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // load u of this wavefront fills LDS bytes [1 KiB (wave INS + u), +1 KiB):
  // lane l -> row 8 (wave INS + u) + l / 8, group position l % 8, holding
  // k-group lq = (l % 8) ^ ((l / 8) & 7)
  const int64_t a_rows = (g.m - m0 < BM) ? (g.m - m0) : BM;
  const i32x4 a_rsrc = make_rsrc(g.a + m0 * g.lda, (uint32_t)(a_rows * g.lda * 2));
  const i32x4 b_rsrc = make_rsrc(g.b + n0 * g.ldb, (uint32_t)(BN * g.ldb * 2));
  const int lr = lane / G, lq = (lane % G) ^ (lr & 7);
  uint32_t a_voff[A_INS];
#pragma unroll
  for (int u = 0; u < A_INS; ++u) {
    int64_t r = 8 * (wave * A_INS + u) + lr;
    if (r >= a_rows) r = a_rows - 1;  // ragged last tile: read a valid row, never store it
    a_voff[u] = (uint32_t)((r * g.lda + 8 * lq) * 2);
  }
  const uint32_t b_voff = (uint32_t)(((8 * wave * B_INS + lr) * g.ldb + 8 * lq) * 2);
  auto issue = [&](int kt, int st) {
    const uint32_t koff = (uint32_t)((int64_t)kt * BK * 2);
#pragma unroll
    for (int u = 0; u < A_INS; ++u)
      buffer_load_lds(a_rsrc, (lds_u32 *)(&As[st][512 * (wave * A_INS + u)]), 16, (int32_t)a_voff[u],
                      (int32_t)koff, 0, 0);
#pragma unroll
    for (int u = 0; u < B_INS; ++u)
      buffer_load_lds(b_rsrc, (lds_u32 *)(&Bs[st][512 * (wave * B_INS + u)]), 16, (int32_t)b_voff,
                      (int32_t)(koff + (uint32_t)(8 * u * g.ldb * 2)), 0, 0);
  };

  f4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  const int row_in = lane & 15, slot = lane >> 4;
  bf16x8 fa[2][FM], fb[2][FN];
  auto fload = [&](int st, int c) {
    const int q = c * 4 + slot;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WM + 16 * i + row_in;
      fa[c][i] = *reinterpret_cast<const bf16x8 *>(&As[st][r * BK + 8 * (q ^ (r & 7))]);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = wn * WN + 16 * j + row_in;
      fb[c][j] = *reinterpret_cast<const bf16x8 *>(&Bs[st][r * BK + 8 * (q ^ (r & 7))]);
    }
  };
  auto mfma_chunk = [&](int c) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[c][i], fb[c][j], acc[i][j], 0, 0, 0);
  };

  issue(0, 0);
  wait_vm0();
  __syncthreads();
  for (int kt = 0; kt < kt_count; ++kt) {
    const int st = kt & 1;
    fload(st, 0);
    if (DEFER && kt > 0) {
      // the previous stage's second chunk, its fragments in registers, covers
      // the latency of this stage's first LDS reads
      __builtin_amdgcn_sched_barrier(0);
      mfma_chunk(1);
      __builtin_amdgcn_sched_barrier(0);
    }
    fload(st, 1);
    // unconditional, so the loop body stays one block: the last iteration
    // reloads its own stage into the idle one, which is never read
    issue(kt + 1 < kt_count ? kt + 1 : kt, st ^ 1);
    mfma_chunk(0);
    if (!DEFER) mfma_chunk(1);
    __builtin_amdgcn_sched_barrier(0);  // the stage's MFMAs stay ahead of the wait
    wait_vm0();                         // this wavefront's loads of the next stage landed
    __syncthreads();                    // everyone's landed; everyone is done reading this stage
  }
  if (DEFER) mfma_chunk(1);

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = m0 + wm * WM + 16 * i + 4 * slot + r;
      if (row < g.m) {
        float *crow = g.c + row * g.ldc + n0 + wn * WN + row_in;
#pragma unroll
        for (int j = 0; j < FN; ++j) crow[16 * j] = acc[i][j][r];
      }
    }
}

template <int BM, int BN, int WM, int WN, int NW, int MINW, bool DEFER>
hipError_t launch(const GemmBf16Args &g, hipStream_t stream) {
  const int64_t m_tiles = (g.m + BM - 1) / BM;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, NW, MINW, DEFER>), dim3((uint32_t)(m_tiles * (g.n / BN))),
                     dim3(NW * 64), 0, stream, g);
  return hipGetLastError();
}

}  // namespace
}  // namespace gemm

// Tile by problem size, as the fp32 projection: 256 x 256 (deferred second
// chunk) with at least 512 tiles, 256 x 128 with at least 256, else 128 x 128
// with two workgroups per CU.
hipError_t launch_gemm_bf16(const GemmBf16Args &g, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  // whole 64-k stages, whole 128-column tiles, tile rows addressable with
  // 32-bit buffer offsets
  if (g.k % gemm::kBKH != 0 || g.n % 128 != 0 || g.lda < g.k || g.ldb < g.k || g.ldc < g.n ||
      (int64_t)256 * g.lda * 2 > INT32_MAX || (int64_t)256 * g.ldb * 2 > INT32_MAX)
    return hipErrorInvalidValue;
  const int64_t m256 = (g.m + 255) / 256;
  if (g.n % 256 == 0 && m256 * (g.n / 256) >= 512) return gemm::launch<256, 256, 64, 128, 8, 1, true>(g, stream);
  if (m256 * (g.n / 128) >= 256) return gemm::launch<256, 128, 64, 64, 8, 1, false>(g, stream);
  return gemm::launch<128, 128, 64, 64, 4, 2, false>(g, stream);
}

}  // namespace kvc
