// Epilogues shared by the prefill projection kernels (the f32 matrix-core
// kernel and the bf16 x f32 three-part kernel). Both use 16 x 16 output
// fragments with the same accumulator layout: accumulator r of lane l holds
// D[4 (l / 16) + r][l % 16].
//
// store_tile: the projection planes, with the positional bias (ape, row =
// token position mod ratio) added to the score half ("DeepSeek V4.1 . Pool
// token pairs", Compressor listing, forward: kv = x wkv^T, score = x wgate^T,
// then score + ape before the softmax).
//
// pool_epilogue: the ratio-4 softmax pooling of the entries whose 8
// candidates lie inside a 256-row tile ("Compressed Sparse Attention . ratio
// m = 4", overlapped blocks: entry j pools branch A of block j and branch B
// of block j - 1, zero / -inf padding before block 0).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gemm_common.h"
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {
namespace gemm {

// Store of one wavefront's FM x FN fragments at rows row0 + .., columns
// col0 + .. of C (row stride g.ldc; row0 a multiple of 4); rows at or past
// g.m are dropped. With bias set, row (row % bias_seqlen) % bias_ratio of it
// is added (bias_ratio a power of two). At ratio 2 or 4 with positions that
// restart at multiples of the ratio (one sequence, or bias_seqlen a multiple
// of the ratio) that row is r % ratio for the lane's r-th row of each group
// of 4, so the lane's 4 x FN bias values are loaded once. Otherwise the
// token position is taken modulo bias_seqlen once per lane and advanced row
// by row, wrapping at bias_seqlen (one wrap at most when bias_seqlen >=
// 16 FM, else each row takes its own modulo).
template <int FM, int FN>
__device__ __forceinline__ void store_tile(const GemmArgs &g, const f4 (&acc)[FM][FN], float *C, const float *bias,
                                           int64_t row0, int64_t col0, int lane) {
  const int row_in = lane & 15, slot = lane >> 4;
  const int64_t seqlen = g.bias_seqlen, ratio = g.bias_ratio;
  if (!bias) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = row0 + 16 * i + 4 * slot + r;
        if (row < g.m) {
          float *crow = C + row * g.ldc + col0 + row_in;
#pragma unroll
          for (int j = 0; j < FN; ++j) crow[16 * j] = acc[i][j][r];
        }
      }
    return;
  }
  if (ratio <= 4 && (g.m <= seqlen || seqlen % ratio == 0)) {
    float bv[4][FN];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < FN; ++j) bv[r][j] = bias[(r & (ratio - 1)) * g.ldc + col0 + row_in + 16 * j];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = row0 + 16 * i + 4 * slot + r;
        if (row < g.m) {
          float *crow = C + row * g.ldc + col0 + row_in;
#pragma unroll
          for (int j = 0; j < FN; ++j) crow[16 * j] = acc[i][j][r] + bv[r][j];
        }
      }
    return;
  }
  const bool one_wrap = seqlen >= 16 * FM;
  const int64_t pos0 = (row0 + 4 * slot) % seqlen;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = row0 + 16 * i + 4 * slot + r;
      if (row < g.m) {
        float *crow = C + row * g.ldc + col0 + row_in;
        int64_t pos;
        if (one_wrap) {
          pos = pos0 + 16 * i + r;
          if (pos >= seqlen) pos -= seqlen;
        } else {
          pos = row % seqlen;
        }
        const float *brow = bias + (pos & (ratio - 1)) * g.ldc + col0 + row_in;
#pragma unroll
        for (int j = 0; j < FN; ++j) crow[16 * j] = acc[i][j][r] + brow[16 * j];
      }
    }
}

// Pooling epilogue of a 256 x 256 tile of WM x WN wavefronts (wm = the
// wavefront's WM-row band, wn its WN columns). Column tile f0 / 64 holds the
// 64 features f0 .. f0 + 63; wavefront column wn the F = WN / 4 features
// f0 + F wn .. +F-1 as four F-column segments: kv branch A (wkv row f), kv
// branch B (wkv row hd + f), score branch A (wgate row f), score branch B
// (wgate row hd + f). A lane's accumulators then hold, for F / 16 features,
// the four rows of one 4-token block of each segment: its own block's branch
// A candidates. The previous block's branch B rows come from the lanes 16
// below (the block above), through LDS (X, kPoolXFloats floats, free for
// reuse: the caller's stage buffers) so that the first block of a wavefront
// reads the wavefront above. Each entry's pooled f32 values go to
// g.pooled, computed by the same softmax code as the pool kernels; the first
// entry of the row tile (whose previous block belongs to another workgroup)
// is pooled afterwards from the plane rows written here: the tile's first
// block (branch A), its last block (branch B) and every row from the last
// complete block of each batch row on (the decode state's source).
constexpr int kPoolXRow = 132;  // 2 x 64 values + 4 pad per row
constexpr int kPoolXFloats = 256 * kPoolXRow;

template <int WM, int WN, bool SIMPLE_PATH = false>
__device__ __forceinline__ void pool_epilogue(const GemmArgs &g, f4 (&acc)[WM / 16][WN / 16], float *X, int64_t m0,
                                              int64_t f0, int wm, int wn, int lane) {
  constexpr int BM = 256, FM = WM / 16, XROW = kPoolXRow;
  constexpr int F = WN / 4, FJ = F / 16;  // features per wavefront, fragments per segment
  static_assert(WN % 64 == 0 && 256 % WM == 0, "pooling wavefront shape");
  const int g4 = lane >> 4, c = lane & 15;
  const int64_t hd = g.pool_hd, seqlen = g.pool_seqlen, groups = g.pool_groups;
  const int64_t gpr = seqlen / 4;  // 4-token blocks per batch row (batch > 1 needs seqlen % 4 == 0)
  // the state's source rows: from the last complete block of each batch row on
  const int64_t state_from = groups > 0 ? 4 * (groups - 1) : 0;
  // the score bias of the lane's features: token position mod 4 is r
  // (blocks start at multiples of 4), the same for every row fragment
  float biasA[4][FJ], biasB[4][FJ];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int jj = 0; jj < FJ; ++jj) {
      const int64_t f = f0 + F * wn + 16 * jj + c;
      biasA[r][jj] = g.bias1 ? g.bias1[r * g.ldc + f] : 0.0f;
      biasB[r][jj] = g.bias1 ? g.bias1[r * g.ldc + hd + f] : 0.0f;
    }
  __syncthreads();  // every wavefront is done with the stage buffers
  // With SIMPLE_PATH, the common case (one sequence, every row of the tile
  // valid, none of them a source row of the decode state) takes a path of
  // its own: the only plane rows stored are the tile's first block (branch
  // A) and its last block (branch B), held by known lanes, so no per-row
  // tests or addresses are needed. It pays where the kernel has registers to
  // spare: the bf16-x kernel's step ran 1.2% faster with it, the f16 one
  // (256 registers) spilled more and ran 1% slower.
  const bool simple = SIMPLE_PATH && g.pool_batch == 1 && m0 + BM <= g.m && m0 + BM <= state_from;
  if (simple) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jj = 0; jj < FJ; ++jj) {
        f4 &kB = acc[i][FJ + jj], &sA = acc[i][2 * FJ + jj], &sB = acc[i][3 * FJ + jj];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (g.bias1) {
            sA[r] = sA[r] + biasA[r][jj];
            sB[r] = sB[r] + biasB[r][jj];
          }
          const int rl = 16 * i + 4 * g4 + r;  // row within the wavefront
          X[(wm * WM + rl) * XROW + wn * 2 * F + 16 * jj + c] = kB[r];
          X[(wm * WM + rl) * XROW + wn * 2 * F + F + 16 * jj + c] = sB[r];
        }
      }
    if (wm == 0 && g4 == 0) {  // rows 0..3 of the tile: fragment 0 of the first band, lanes 0..15
#pragma unroll
      for (int jj = 0; jj < FJ; ++jj) {
        const int64_t f = f0 + F * wn + 16 * jj + c;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          g.c0[(m0 + r) * g.ldc + f] = acc[0][jj][r];
          g.c1[(m0 + r) * g.ldc + f] = acc[0][2 * FJ + jj][r];
        }
      }
    }
    if (wm == BM / WM - 1 && g4 == 3) {  // rows BM-4..BM-1: last fragment of the last band, lanes 48..63
#pragma unroll
      for (int jj = 0; jj < FJ; ++jj) {
        const int64_t f = f0 + F * wn + 16 * jj + c;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          g.c0[(m0 + BM - 4 + r) * g.ldc + hd + f] = acc[FM - 1][FJ + jj][r];
          g.c1[(m0 + BM - 4 + r) * g.ldc + hd + f] = acc[FM - 1][3 * FJ + jj][r];
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jj = 0; jj < FJ; ++jj) {
        const int64_t f = f0 + F * wn + 16 * jj + c;
        f4 &kA = acc[i][jj], &kB = acc[i][FJ + jj], &sA = acc[i][2 * FJ + jj], &sB = acc[i][3 * FJ + jj];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rl = 16 * i + 4 * g4 + r;  // row within the wavefront
          const int64_t row = m0 + wm * WM + rl;
          if (g.bias1) {
            sA[r] = sA[r] + biasA[r][jj];
            sB[r] = sB[r] + biasB[r][jj];
          }
          if (row < g.m) {
            const int64_t tpos = g.pool_batch == 1 ? row : row % seqlen;
            const int tile_row = wm * WM + rl;
            const bool state_row = tpos >= state_from;
            float *kv = g.c0 + row * g.ldc, *sc = g.c1 + row * g.ldc;
            if (state_row || tile_row < 4) {  // branch A: state rows and the tile's first block
              kv[f] = kA[r];
              sc[f] = sA[r];
            }
            if (state_row || tile_row >= BM - 4) {  // branch B: state rows and the tile's last block
              kv[hd + f] = kB[r];
              sc[hd + f] = sB[r];
            }
          }
          X[(wm * WM + rl) * XROW + wn * 2 * F + 16 * jj + c] = kB[r];
          X[(wm * WM + rl) * XROW + wn * 2 * F + F + 16 * jj + c] = sB[r];
        }
      }
  }
  __syncthreads();  // branch B of every block is in LDS
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t gf = (m0 + wm * WM + 16 * i) / 4 + g4;  // 4-token block of the flattened rows
    const int64_t b = g.pool_batch == 1 ? 0 : gf / gpr;
    const int64_t j = g.pool_batch == 1 ? gf : gf - b * gpr;
    // entries of complete blocks; the row tile's first entry needs the
    // previous workgroup's block and is pooled afterwards (unless it is
    // its batch row's entry 0, whose previous block is padding)
    const bool first_of_tile = wm == 0 && i == 0 && g4 == 0;
    if (b >= g.pool_batch || j >= groups || (first_of_tile && j > 0)) continue;
    // the previous block's rows in LDS: 4 rows up, into the wavefront above
    const int prow = wm * WM + 16 * i + 4 * g4 - 4;
#pragma unroll
    for (int jj = 0; jj < FJ; ++jj) {
      float ck[8][1], cs[8][1];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (j == 0) {
          ck[r][0] = 0.0f;
          cs[r][0] = -INFINITY;
        } else {
          ck[r][0] = X[(prow + r) * XROW + wn * 2 * F + 16 * jj + c];
          cs[r][0] = X[(prow + r) * XROW + wn * 2 * F + F + 16 * jj + c];
        }
        ck[4 + r][0] = acc[i][jj][r];
        cs[4 + r][0] = acc[i][2 * FJ + jj][r];
      }
      float p[1];
      softmax_pool<8, 1>(ck, cs, p);
      g.pooled[(b * groups + j) * hd + f0 + F * wn + 16 * jj + c] = p[0];
    }
  }
}

}  // namespace gemm
}  // namespace kvc
