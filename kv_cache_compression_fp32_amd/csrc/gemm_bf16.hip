// bf16 matrix-core GEMMs of the compressor's projections (gfx950, wave64).
//
// 1. Prefill projection for bf16 hidden states: C = x . w^T with x bf16 and
//    w f32, computed on the bf16 matrix cores without rounding anything but
//    the f32 accumulation. "DeepSeek V4.1 . Pool token pairs", Compressor
//    listing, forward: the model's hidden state x (bf16) is promoted to f32
//    and multiplied by the f32 wkv / wgate ("Module compress", Functions,
//    linear_f32). The promotion is exact, and every f32 weight is the exact
//    sum of three bf16 values:
//      hi = w with its low 16 bits cleared, mid = (w - hi) with its low 16
//      bits cleared, lo = w - hi - mid.
//    (w - hi and w - hi - mid are exact f32 differences; the bits of w below
//    hi number 16, so mid takes the top 8 significant ones and lo the at
//    most 8 left, which a bf16 holds exactly. Clearing bits never rounds up,
//    so no part overflows.) Each bf16 x bf16 product is exact in f32, and
//      x . w = x . hi + x . mid + x . lo
//    term by term, so three bf16 matrix-core passes with f32 accumulation
//    give the f32 product with no error beyond the accumulation's own
//    rounding, in K / 32 * 3 accumulation steps per output (the f32
//    instruction takes K / 4). split_weights_kernel writes the parts as
//    bsplit[2 n_half][3][k] (wkv rows, then wgate rows); for the pooling
//    kernel the rows are permuted into the order its column tiles read
//    (pool_epilogue, gemm_epilogue.h).
// 2. The ratio-1 projection (bf16 x times bf16 wkv, f32 accumulation; the
//    Compressor listing's __init__ and ratio-1 branch of forward; "Module
//    compress", CompressorWeights): the same kernel with plain bf16 weights.
//
// gemm_mc_kernel: BM x BN workgroup tile, WM x WN per wavefront, two LDS
// stages of 64 KiB: with the split weights, one 32-k slice of the x tile
// [BM][32] and the three weight parts [3][BN][32]; with plain weights, two
// 32-k slices of each. Slices are 64-byte rows of four 8-bf16 k-groups,
// group q of row r at position q ^ ((r / 2) & 3) (the 16-byte reads of 8
// neighbouring rows hit 8 distinct 16-byte bank groups). Loads are buffer
// loads that write LDS directly, 16 rows x 32 k (1 KiB) per instruction.
// Matrix-core layout (v_mfma_f32_16x16x32_bf16, lane l): 8 consecutive k of
// row l % 16, k-group l / 16; accumulator r holds D[4 (l / 16) + r][l % 16],
// as in the f32 kernel.
//
// Schedule ("ping-pong"): the 8 wavefronts form two groups, 0..3 and 4..7,
// so that every SIMD holds one wavefront of each. Both groups run the same
// loop, phase by phase with a barrier between phases: read a stage's
// fragments from LDS, then run its MFMAs from registers. Group 4..7 starts
// one phase late, so on every SIMD one wavefront multiplies while the other
// reads: the matrix cores do not wait for the barrier's stragglers or the
// first LDS reads after it. Group 0..3 alone issues the global -> LDS loads,
// each stage's loads right after its reads of the previous stage (so no LDS
// read of the group follows a load in flight), and waits for them at the
// end of its multiply phase, before the barrier after which it reads them.
// Buffer reuse: a stage buffer is reloaded one phase after group 4..7 read
// it; that group waits for its own LDS reads before each barrier. Every
// wavefront meets the same 2 k / (k per stage) + 2 barriers.
#include "gemm_common.h"
#include "gemm_epilogue.h"
#include "kvc_launch.h"

namespace kvc {
namespace gemm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// A workgroup barrier without the memory fence of __syncthreads (which would
// also wait for the loading group's loads in flight), kept in place by the
// scheduler; the waits each phase needs are explicit.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

constexpr int kBK3 = 32;  // k per LDS stage
// the pooling kernel's wavefront: 128 rows x 64 columns, the 64 columns the
// four 16-wide segments (kvA, kvB, scA, scB) of 16 features
constexpr int kPoolWM = 128, kPoolWN = 64, kPoolF = kPoolWN / 4;

// one thread per 8 consecutive k of one output row
__global__ __launch_bounds__(256) void split_weights_kernel(SplitArgs a) {
  const int64_t per_row = a.k / 8;
  const int64_t total = 2 * a.n_half * per_row;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t row = i / per_row, k0 = 8 * (i - row * per_row);
  const float *src;
  if (a.pool_hd) {
    // pooling order: column tile t = row / T (T = pool_tile rows) holds
    // features T / 4 t .. +T / 4 - 1; within it, [T / 64 wavefront
    // columns][kvA, kvB, scA, scB][16 features]
    const int64_t T = a.pool_tile;
    const int64_t t = row / T, rem = row % T, wn = rem / (4 * kPoolF), seg = (rem % (4 * kPoolF)) / kPoolF,
                  c = rem % kPoolF;
    const int64_t f = (T / 4) * t + kPoolF * wn + c;
    src = (seg < 2 ? a.w0 : a.w1) + ((seg & 1) * a.pool_hd + f) * a.ldw;
  } else {
    src = row < a.n_half ? a.w0 + row * a.ldw : a.w1 + (row - a.n_half) * a.ldw;
  }
  const float4 v0 = *reinterpret_cast<const float4 *>(src + k0);
  const float4 v1 = *reinterpret_cast<const float4 *>(src + k0 + 4);
  const float w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint32_t hi[4], mid[4], lo[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    uint32_t h2[2], m2[2], l2[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t hb = __float_as_uint(w[e + u]) & 0xffff0000u;
      const float r1 = w[e + u] - __uint_as_float(hb);
      const uint32_t mb = __float_as_uint(r1) & 0xffff0000u;
      const float r2 = r1 - __uint_as_float(mb);
      h2[u] = hb >> 16;
      m2[u] = mb >> 16;
      l2[u] = __float_as_uint(r2) >> 16;
    }
    hi[e / 2] = h2[0] | (h2[1] << 16);
    mid[e / 2] = m2[0] | (m2[1] << 16);
    lo[e / 2] = l2[0] | (l2[1] << 16);
  }
  uint16_t *dst = a.out + row * 3 * a.k + k0;
  *reinterpret_cast<uint4 *>(dst) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  *reinterpret_cast<uint4 *>(dst + a.k) = make_uint4(mid[0], mid[1], mid[2], mid[3]);
  *reinterpret_cast<uint4 *>(dst + 2 * a.k) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

// SPLIT3: a stage is one 32-k slice of x times the three parts of the split
// weights of the same k (g.bsplit, rows of 3 k: hi, mid, lo), two output
// halves (c0, c1). Otherwise (the ratio-1 projection) a stage is two 32-k
// slices of x times the same two slices of bf16 weights (g.bsplit = the
// weights, row stride ldb), one output plane c0 of n_half columns. Either
// way a stage holds 64 KiB and every output sums its k in increasing order.
template <int BM, int BN, int WM, int WN, int NW, int MINW, bool POOL, bool SPLIT3>
__global__ __launch_bounds__(NW * 64, MINW) void gemm_mc_kernel(GemmArgs g) {
  constexpr int BK = kBK3;              // k per slice
  constexpr int XS = SPLIT3 ? 1 : 2;    // x slices per stage
  constexpr int WS = SPLIT3 ? 3 : 2;    // weight slices per stage: parts, or k slices
  constexpr int KPS = XS * BK;          // k per stage
  constexpr int WAVES_N = BN / WN;
  static_assert((BM / WM) * (BN / WN) == NW, "wavefront grid must cover the tile");
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int ARB = BM / 16, BRB = BN / 16;  // 16-row load blocks per slice
  static_assert(NW == 8, "two groups of four wavefronts");
  constexpr int NL = 4;  // loading wavefronts (group 0..3)
  constexpr int A_INS = XS * ARB / NL, B_INS = WS * BRB / NL;  // 1 KiB loads per loading wavefront
  static_assert(A_INS * NL == XS * ARB && B_INS * NL == WS * BRB, "tile/wavefront mismatch");
  static_assert(!POOL || (SPLIT3 && BM == 256 && BN == 256 && WM == kPoolWM && WN == kPoolWN && NW == 8),
                "pooling tile shape");
  // stage buffers as floats (x slices then weight slices), reused by the pooling epilogue
  constexpr int STAGE_FLOATS = 2 * (XS * BM + WS * BN) * BK / 2;
  constexpr int SMEM_FLOATS = POOL && kPoolXFloats > STAGE_FLOATS ? kPoolXFloats : STAGE_FLOATS;
  __shared__ __attribute__((aligned(16))) float smem[SMEM_FLOATS];
  uint16_t(*As)[XS][BM * BK] = reinterpret_cast<uint16_t(*)[XS][BM * BK]>(smem);
  uint16_t(*Bs)[WS][BN * BK] = reinterpret_cast<uint16_t(*)[WS][BN * BK]>(smem + XS * BM * BK);

  const int64_t m_tiles = (g.m + BM - 1) / BM;
  // with POOL: pool_hd / 64 tiles of 256 permuted rows
  const int64_t n_tiles = (SPLIT3 ? 2 * g.n_half : g.n_half) / BN;
  const uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t mt = tile / n_tiles, nt = tile - mt * n_tiles;
  if (mt >= m_tiles) return;
  const int64_t m0 = mt * BM;
  const int64_t n_glob = nt * BN;
  const bool second = n_glob >= g.n_half;
  const int64_t n0 = second ? n_glob - g.n_half : n_glob;
  const int kt_count = (int)(g.k / KPS);

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  // the wavefront index as a scalar: the loads' LDS addresses and offsets
  // derived from it are then wavefront-uniform values, not per-lane ones
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool loader = wave_u < NL;  // group 0..3
  const int lw = wave_u % NL;       // its index among the loading wavefronts

  // Load u of this wavefront fills 1 KiB = 16 rows of 64 bytes: lane l ->
  // row l / 4 of the block, group position l % 4, which holds k-group
  // lq = (l % 4) ^ (((l / 4) / 2) & 3). The x resource starts at the tile's
  // first row, the weight resource at the tile's first weight row (row
  // stride RS); x load q covers slice q / ARB, rows 16 (q % ARB) ..; weight
  // load q covers slice q / BRB (at element offset PS apart), rows
  // 16 (q % BRB) ..; slice, row block and k offsets are wavefront-uniform
  // (soffset) for the weights.
  const int64_t RS = SPLIT3 ? 3 * g.k : g.ldb, PS = SPLIT3 ? g.k : BK;
  const int64_t a_rows = (g.m - m0 < BM) ? (g.m - m0) : BM;
  const i32x4 a_rsrc = make_rsrc(g.a16 + m0 * g.lda, (uint32_t)(a_rows * g.lda * 2));
  const i32x4 b_rsrc = make_rsrc(g.bsplit + n_glob * RS, (uint32_t)(BN * RS * 2));
  const int lr = lane >> 2, lq = (lane & 3) ^ ((lr >> 1) & 3);
  uint32_t a_voff[A_INS];
#pragma unroll
  for (int u = 0; u < A_INS; ++u) {
    const int q = lw * A_INS + u;
    int64_t r = 16 * (q % ARB) + lr;
    if (r >= a_rows) r = a_rows - 1;  // ragged last tile: read a valid row, never store it
    a_voff[u] = (uint32_t)((r * g.lda + (q / ARB) * BK + 8 * lq) * 2);
  }
  const uint32_t b_voff = (uint32_t)((lr * RS + 8 * lq) * 2);
  auto issue = [&](int kt, int st) {
    const uint32_t koff = (uint32_t)(kt * KPS * 2);
#pragma unroll
    for (int u = 0; u < A_INS; ++u) {
      const int q = lw * A_INS + u;
      buffer_load_lds(a_rsrc, (lds_u32 *)(&As[st][q / ARB][512 * (q % ARB)]), 16, (int32_t)a_voff[u],
                      (int32_t)koff, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < B_INS; ++u) {
      const int q = lw * B_INS + u, p = q / BRB, rb = q % BRB;
      buffer_load_lds(b_rsrc, (lds_u32 *)(&Bs[st][p][512 * rb]), 16, (int32_t)b_voff,
                      (int32_t)(koff + (uint32_t)((rb * 16 * RS + p * PS) * 2)), 0, 0);
    }
  };

  f4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  const int row_in = lane & 15, slot = lane >> 4;
  bf16x8 fa[XS][FM], fb[WS][FN];
  auto reads = [&](int st) {
#pragma unroll
    for (int s = 0; s < XS; ++s)
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WM + 16 * i + row_in;
        fa[s][i] = *reinterpret_cast<const bf16x8 *>(&As[st][s][r * BK + 8 * (slot ^ ((r >> 1) & 3))]);
      }
#pragma unroll
    for (int p = 0; p < WS; ++p)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WN + 16 * j + row_in;
        fb[p][j] = *reinterpret_cast<const bf16x8 *>(&Bs[st][p][r * BK + 8 * (slot ^ ((r >> 1) & 3))]);
      }
  };
  auto mfmas = [&]() {  // SPLIT3: hi, then mid, then lo; else the two k slices in order
#pragma unroll
    for (int p = 0; p < WS; ++p)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[SPLIT3 ? 0 : p][i], fb[p][j], acc[i][j], 0, 0, 0);
  };

  if (loader) {
    issue(0, 0);
    wait_vm0();
  }
  phase_barrier();
  if (!loader) phase_barrier();  // group 4..7 runs one phase behind
  for (int kt = 0; kt < kt_count; ++kt) {
    const int st = kt & 1;
    reads(st);
    if (loader && kt + 1 < kt_count) issue(kt + 1, st ^ 1);  // after the stage's last LDS read
    wait_lgkm0();  // this stage's reads are done before its buffer can be reloaded
    phase_barrier();
    mfmas();
    if (loader) wait_vm0();  // the next stage has landed before this group reads it
    phase_barrier();
  }
  if (loader) phase_barrier();  // the same number of barriers for every wavefront

  if constexpr (POOL) {
    pool_epilogue<WM, WN>(g, acc, smem, m0, 64 * nt, wm, wn, lane);
  } else {
    store_tile<FM, FN>(g, acc, second ? g.c1 : g.c0, second ? g.bias1 : nullptr, m0 + wm * WM, n0 + wn * WN,
                       lane);
  }
}


// f32 x times the three-part weights: gemm_x6_kernel. A 256 x 128 tile of
// eight 64 x 64 wavefronts, the same ping-pong schedule and weight slices as
// gemm_mc_kernel; the x tile stays f32 in LDS ([256][32] floats per stage,
// 16-byte k-group q of row r at position q ^ (r & 7), loaded 8 rows per
// instruction as in the f32 kernel). The read phase splits each x fragment
// (8 consecutive k of a row) like the weights, x = xh + xm + xl (exact, bits
// cleared), and the multiply phase sums the six part products whose size is
// at least 2^-16 |x w|: xh wh, xh wm, xm wh, xh wl, xm wm, xl wh. The three
// left out (xm wl, xl wm, xl wl) are below 2^-21 |x w| together, far inside
// the f32 summation's own error bound (K 2^-24 sum |x w|).
__device__ __forceinline__ void split8(const f4 lo4, const f4 hi4, bf16x8 &h, bf16x8 &m, bf16x8 &l) {
  const float v[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
  uint32_t hw[4], mw[4], lw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t hb[2], mb[2], lb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t b = __float_as_uint(v[2 * e + u]);
      hb[u] = b & 0xffff0000u;
      const float r1 = v[2 * e + u] - __uint_as_float(hb[u]);
      mb[u] = __float_as_uint(r1) & 0xffff0000u;
      lb[u] = __float_as_uint(r1 - __uint_as_float(mb[u]));  // exact: its low 16 bits are zero
    }
    hw[e] = (hb[0] >> 16) | hb[1];
    mw[e] = (mb[0] >> 16) | mb[1];
    lw[e] = (lb[0] >> 16) | lb[1];
  }
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const u4 hv = {hw[0], hw[1], hw[2], hw[3]}, mv = {mw[0], mw[1], mw[2], mw[3]}, lv = {lw[0], lw[1], lw[2], lw[3]};
  h = __builtin_bit_cast(bf16x8, hv);
  m = __builtin_bit_cast(bf16x8, mv);
  l = __builtin_bit_cast(bf16x8, lv);
}

template <bool POOL>
__global__ __launch_bounds__(512, 1) void gemm_x6_kernel(GemmArgs g) {
  constexpr int BM = 256, BN = 128, WM = 64, WN = 64, BK = kBK3;
  constexpr int WAVES_N = BN / WN;  // 2
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int BRB = BN / 16;
  constexpr int NL = 4;
  constexpr int A_INS = BM / 8 / NL, B_INS = 3 * BRB / NL;  // x: 8 rows of 32 floats per load
  constexpr int STAGE_FLOATS = 2 * (BM * BK + 3 * BN * BK / 2);
  constexpr int SMEM_FLOATS = POOL && kPoolXFloats > STAGE_FLOATS ? kPoolXFloats : STAGE_FLOATS;
  __shared__ __attribute__((aligned(16))) float smem[SMEM_FLOATS];
  float(*As)[BM * BK] = reinterpret_cast<float(*)[BM * BK]>(smem);
  uint16_t(*Bs)[3][BN * BK] = reinterpret_cast<uint16_t(*)[3][BN * BK]>(smem + 2 * BM * BK);

  const int64_t m_tiles = (g.m + BM - 1) / BM;
  const int64_t n_tiles = 2 * g.n_half / BN;  // with POOL: pool_hd / 32 tiles of 128 permuted rows
  const uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t mt = tile / n_tiles, nt = tile - mt * n_tiles;
  if (mt >= m_tiles) return;
  const int64_t m0 = mt * BM, n_glob = nt * BN;
  const bool second = n_glob >= g.n_half;
  const int64_t n0 = second ? n_glob - g.n_half : n_glob;
  const int kt_count = (int)(g.k / BK);

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool loader = wave_u < NL;
  const int lw = wave_u % NL;

  // x: load u of a loading wavefront fills rows 8 (lw A_INS + u) .. +7,
  // lane l -> row l / 8, group position l % 8 holding k-group
  // (l % 8) ^ ((l / 8) & 7); weights as gemm_mc_kernel (rows of 3 k).
  const int64_t RS = 3 * g.k;
  const int64_t a_rows = (g.m - m0 < BM) ? (g.m - m0) : BM;
  const i32x4 a_rsrc = make_rsrc(g.a + m0 * g.lda, (uint32_t)(a_rows * g.lda * 4));
  const i32x4 b_rsrc = make_rsrc(g.bsplit + n_glob * RS, (uint32_t)(BN * RS * 2));
  const int xr = lane >> 3, xq = (lane & 7) ^ (xr & 7);
  uint32_t a_voff[A_INS];
#pragma unroll
  for (int u = 0; u < A_INS; ++u) {
    int64_t r = 8 * (lw * A_INS + u) + xr;
    if (r >= a_rows) r = a_rows - 1;  // ragged last tile: read a valid row, never store it
    a_voff[u] = (uint32_t)((r * g.lda + 4 * xq) * 4);
  }
  const int lr = lane >> 2, lq = (lane & 3) ^ ((lr >> 1) & 3);
  const uint32_t b_voff = (uint32_t)((lr * RS + 8 * lq) * 2);
  auto issue = [&](int kt, int st) {
#pragma unroll
    for (int u = 0; u < A_INS; ++u)
      buffer_load_lds(a_rsrc, (lds_u32 *)(&As[st][256 * (lw * A_INS + u)]), 16, (int32_t)a_voff[u],
                      (int32_t)(kt * BK * 4), 0, 0);
#pragma unroll
    for (int u = 0; u < B_INS; ++u) {
      const int q = lw * B_INS + u, p = q / BRB, rb = q % BRB;
      buffer_load_lds(b_rsrc, (lds_u32 *)(&Bs[st][p][512 * rb]), 16, (int32_t)b_voff,
                      (int32_t)((uint32_t)(kt * BK * 2) + (uint32_t)((rb * 16 * RS + p * g.k) * 2)), 0, 0);
    }
  };

  f4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  const int row_in = lane & 15, slot = lane >> 4;
  // the read phase keeps x as f32 (8 values per row fragment) and splits row
  // fragment 0; the multiply phase splits row fragment i + 1 while row
  // fragment i's MFMAs run
  f4 xf[FM][2];
  bf16x8 fa[2][3], fb[3][FN];
  auto reads = [&](int st) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WM + 16 * i + row_in;
      xf[i][0] = *reinterpret_cast<const f4 *>(&As[st][r * BK + 4 * ((2 * slot) ^ (r & 7))]);
      xf[i][1] = *reinterpret_cast<const f4 *>(&As[st][r * BK + 4 * ((2 * slot + 1) ^ (r & 7))]);
    }
#pragma unroll
    for (int p = 0; p < 3; ++p)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WN + 16 * j + row_in;
        fb[p][j] = *reinterpret_cast<const bf16x8 *>(&Bs[st][p][r * BK + 8 * (slot ^ ((r >> 1) & 3))]);
      }
    // row fragment 0 split here, so the multiply phase opens with MFMAs
    split8(xf[0][0], xf[0][1], fa[0][0], fa[0][1], fa[0][2]);
  };
  // per row fragment, the six part products in the order xh wh, xh wm,
  // xm wh, xh wl, xm wm, xl wh (every output sums them in that order)
  auto mfmas = [&]() {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int cur = i & 1;
      if (i + 1 < FM) split8(xf[i + 1][0], xf[i + 1][1], fa[cur ^ 1][0], fa[cur ^ 1][1], fa[cur ^ 1][2]);
      constexpr int XP[6] = {0, 0, 1, 0, 1, 2}, WP[6] = {0, 1, 0, 2, 1, 0};
#pragma unroll
      for (int q = 0; q < 6; ++q)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[cur][XP[q]], fb[WP[q]][j], acc[i][j], 0, 0, 0);
    }
  };

  if (loader) {
    issue(0, 0);
    wait_vm0();
  }
  phase_barrier();
  if (!loader) phase_barrier();  // group 4..7 runs one phase behind
  for (int kt = 0; kt < kt_count; ++kt) {
    const int st = kt & 1;
    reads(st);
    if (loader && kt + 1 < kt_count) issue(kt + 1, st ^ 1);  // after the stage's last LDS read
    wait_lgkm0();
    phase_barrier();
    mfmas();
    if (loader) wait_vm0();
    phase_barrier();
  }
  if (loader) phase_barrier();  // the same number of barriers for every wavefront

  if constexpr (POOL) {
    pool_epilogue<WM, WN>(g, acc, smem, m0, 32 * nt, wm, wn, lane);
  } else {
    store_tile<FM, FN>(g, acc, second ? g.c1 : g.c0, second ? g.bias1 : nullptr, m0 + wm * WM, n0 + wn * WN,
                       lane);
  }
}

template <int BM, int BN, int WM, int WN, int NW, int MINW, bool POOL, bool SPLIT3 = true>
hipError_t launch(const GemmArgs &g, int64_t n_tiles, hipStream_t stream) {
  const int64_t m_tiles = (g.m + BM - 1) / BM;
  hipLaunchKernelGGL((gemm_mc_kernel<BM, BN, WM, WN, NW, MINW, POOL, SPLIT3>), dim3((uint32_t)(m_tiles * n_tiles)),
                     dim3(NW * 64), 0, stream, g);
  return hipGetLastError();
}

// whole stages, and rows of x and of the weights addressable with 32-bit
// buffer offsets (weight rows of `row_elems` bf16 values)
bool addressable(const GemmArgs &g, int64_t k_per_stage, int64_t row_elems) {
  return g.lda >= g.k && g.k % k_per_stage == 0 && (int64_t)256 * g.lda * 2 <= INT32_MAX &&
         256 * row_elems * 2 <= INT32_MAX;
}

}  // namespace
}  // namespace gemm

hipError_t launch_split_weights(const SplitArgs &a, hipStream_t stream) {
  if (a.n_half <= 0 || a.k <= 0) return hipSuccess;
  if (a.k % 8 != 0 || a.ldw < a.k || (a.pool_hd && 2 * a.n_half != 4 * (int64_t)a.pool_hd) ||
      (a.pool_hd && (a.pool_tile != 256 && a.pool_tile != 128)) || (a.pool_hd && a.pool_hd % (a.pool_tile / 4) != 0))
    return hipErrorInvalidValue;
  const int64_t total = 2 * a.n_half * (a.k / 8);
  hipLaunchKernelGGL(gemm::split_weights_kernel, dim3((uint32_t)((total + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// 256 x 256 tiles (eight 128 x 64 wavefronts: the taller wavefront reads
// fewer weight fragments, which come in three parts) when the column tiles
// fit the halves, else 256 x 128 (eight 64 x 64 wavefronts).
hipError_t launch_gemm_x3(const GemmArgs &g, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  if (g.n_half % 128 != 0 || !gemm::addressable(g, gemm::kBK3, 3 * g.k) ||
      (g.bias1 && (g.bias_seqlen < 1 || g.bias_ratio < 1 || (g.bias_ratio & (g.bias_ratio - 1)) != 0)))
    return hipErrorInvalidValue;
  if (g.n_half % 256 == 0) return gemm::launch<256, 256, 128, 64, 8, 1, false>(g, 2 * g.n_half / 256, stream);
  return gemm::launch<256, 128, 64, 64, 8, 1, false>(g, 2 * g.n_half / 128, stream);
}

hipError_t launch_gemm_x3_pool(const GemmArgs &g, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  // 64-feature column tiles, 4-token blocks aligned with the flattened rows
  if (g.pool_hd % 64 != 0 || g.n_half != 2 * (int64_t)g.pool_hd || g.ldc != 2 * g.pool_hd ||
      !gemm::addressable(g, gemm::kBK3, 3 * g.k) || g.m != g.pool_batch * g.pool_seqlen ||
      (g.pool_batch > 1 && g.pool_seqlen % 4 != 0) || !g.pooled)
    return hipErrorInvalidValue;
  return gemm::launch<256, 256, gemm::kPoolWM, gemm::kPoolWN, 8, 1, true>(g, g.pool_hd / 64, stream);
}

}  // namespace kvc

namespace kvc {

// The ratio-1 projection: bf16 x times bf16 weights, the same kernel with two
// k slices per stage; 256 x 256 tiles when the columns allow, else 256 x 128.
hipError_t launch_gemm_bf16(const GemmBf16Args &a, hipStream_t stream) {
  if (a.m <= 0) return hipSuccess;
  GemmArgs g{};
  g.a16 = a.a;
  g.bsplit = a.b;
  g.c0 = a.c;
  g.lda = a.lda;
  g.ldb = a.ldb;
  g.ldc = a.ldc;
  g.m = a.m;
  g.n_half = a.n;
  g.k = a.k;
  if (a.n % 128 != 0 || a.ldb < a.k || a.ldc < a.n || !gemm::addressable(g, 2 * gemm::kBK3, a.ldb))
    return hipErrorInvalidValue;
  if (a.n % 256 == 0) return gemm::launch<256, 256, 128, 64, 8, 1, false, false>(g, a.n / 256, stream);
  return gemm::launch<256, 128, 64, 64, 8, 1, false, false>(g, a.n / 128, stream);
}

}  // namespace kvc

namespace kvc {

hipError_t launch_gemm_x6(const GemmArgs &g, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  if (g.n_half % 128 != 0 || g.lda < g.k || g.k % gemm::kBK3 != 0 || (int64_t)256 * g.lda * 4 > INT32_MAX ||
      (int64_t)128 * 3 * g.k * 2 > INT32_MAX ||
      (g.bias1 && (g.bias_seqlen < 1 || g.bias_ratio < 1 || (g.bias_ratio & (g.bias_ratio - 1)) != 0)))
    return hipErrorInvalidValue;
  const int64_t m_tiles = (g.m + 255) / 256;
  hipLaunchKernelGGL(gemm::gemm_x6_kernel<false>, dim3((uint32_t)(m_tiles * (2 * g.n_half / 128))), dim3(512), 0,
                     stream, g);
  return hipGetLastError();
}

hipError_t launch_gemm_x6_pool(const GemmArgs &g, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  if (g.pool_hd % 32 != 0 || g.n_half != 2 * (int64_t)g.pool_hd || g.ldc != 2 * g.pool_hd || g.lda < g.k ||
      g.k % gemm::kBK3 != 0 || (int64_t)256 * g.lda * 4 > INT32_MAX || (int64_t)128 * 3 * g.k * 2 > INT32_MAX ||
      g.m != g.pool_batch * g.pool_seqlen || (g.pool_batch > 1 && g.pool_seqlen % 4 != 0) || !g.pooled)
    return hipErrorInvalidValue;
  const int64_t m_tiles = (g.m + 255) / 256;
  hipLaunchKernelGGL(gemm::gemm_x6_kernel<true>, dim3((uint32_t)(m_tiles * (g.pool_hd / 32))), dim3(512), 0, stream,
                     g);
  return hipGetLastError();
}

}  // namespace kvc
