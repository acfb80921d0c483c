// 16-bit matrix-core GEMMs of the compressor's projections (gfx950, wave64):
// the f32 products x . w^T ("Module compress", Functions, linear_f32) from
// parts of the f32 operands, and the ratio-1 bf16 projection.
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
// 3. Opt-in emulations of the prefill projection for f32 hidden states (the
//    default for them is the f32 matrix cores, gemm_f32_kernel.h):
//    gemm_x6_kernel, with x split in registers, either like the weights into
//    three bf16 parts (six part products, KVC_PROJ_BF16_SPLIT) or into two
//    f16 parts of the row scaled by a power of two, against the weights' two
//    f16 parts (KVC_PROJ_F16_SPLIT: split_weights_f16_kernel,
//    row_exponents_kernel; three part products, the sums scaled back
//    exactly).
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
#include <type_traits>

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
// Counter waits as s_waitcnt instructions the compiler sees (so it knows the
// counters drained there and adds no waits of its own for earlier loads, as
// it would after an opaque asm wait), kept in place by the scheduler.
// Immediate fields: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void wait_vm0_seen() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
}

// vmcnt(1): every load but the last one issued has landed (loads land in
// the order they were issued)
__device__ __forceinline__ void wait_vm1_seen() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F71);  // vmcnt(1)
  __builtin_amdgcn_sched_barrier(0);
}

// f32 x tiles: the x lines of the stage after the one being loaded are
// touched too (one 4-byte load per 128-byte line, landing in a scratch LDS
// row), so that they are on their way to L2 one step before the stage load
// asks for them; with two LDS stages the stage load itself has only one
// multiply phase to arrive. Stages ahead of the stage load (0: off).
constexpr int kXPrefetch = 1;

constexpr int kBK3 = 32;  // k per LDS stage
// the pooling kernel's wavefront: 128 rows x 64 columns, the 64 columns the
// four 16-wide segments (kvA, kvB, scA, scB) of 16 features
constexpr int kPoolWM = 128, kPoolWN = 64, kPoolF = kPoolWN / 4;

// Source weight row of split row `row`. Pooling order: column tile
// t = row / T (T = pool_tile rows) holds features T / 4 t .. +T / 4 - 1;
// within it, [T / W wavefront columns][kvA, kvB, scA, scB][W / 4 features]
// (W = pool_wn, the wavefront's columns).
__device__ __forceinline__ const float *split_source_row(const SplitArgs &a, int64_t row) {
  if (a.pool_hd) {
    const int64_t T = a.pool_tile, W = a.pool_wn, F = W / 4;
    const int64_t t = row / T, rem = row % T, wn = rem / W, seg = (rem % W) / F, c = rem % F;
    const int64_t f = (T / 4) * t + F * wn + c;
    return (seg < 2 ? a.w0 : a.w1) + ((seg & 1) * a.pool_hd + f) * a.ldw;
  }
  return row < a.n_half ? a.w0 + row * a.ldw : a.w1 + (row - a.n_half) * a.ldw;
}

// one thread per 8 consecutive k of one output row
__global__ __launch_bounds__(256) void split_weights_kernel(SplitArgs a) {
  const int64_t per_row = a.k / 8;
  const int64_t total = 2 * a.n_half * per_row;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t row = i / per_row, k0 = 8 * (i - row * per_row);
  const float *src = split_source_row(a, row);
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

// f16 parts. A row (of x, or a weight row) is scaled by 2^e so that its
// largest magnitude lies in [2^14, 2^15), inside the f16 range; a scaled
// value y splits into h = f16(y) and l = f16(y - h), both rounded to nearest
// even. y - h is exact in f32 (the bits of y below h's last place), so
// |y - h - l| <= 2^-22 |y|, or at most 2^-25 (2^-40 of the row's largest
// magnitude, unscaled) where l lies below the f16 normal range.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int f16_row_exponent(float amax) {
  if (!(amax > 0.0f) || !(amax < INFINITY)) return 0;  // zeros, infinities
  return 15 - __builtin_amdgcn_frexp_expf(amax);         // amax in [2^(E-1), 2^E)
}

__device__ __forceinline__ void split_f16(float v, int e, _Float16 &h, _Float16 &l) {
  const float y = __builtin_amdgcn_ldexpf(v, e);
  h = (_Float16)y;
  l = (_Float16)(y - (float)h);
}

__device__ __forceinline__ float block_max_256(float v) {
  __shared__ float part[4];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
}

// one workgroup of 256 per split row: the row's largest magnitude, then the
// two f16 parts of the scaled row (h at out + 2 k row, l at + k)
__global__ __launch_bounds__(256) void split_weights_f16_kernel(SplitArgs a) {
  const int64_t row = blockIdx.x;
  const float *src = split_source_row(a, row);
  float amax = 0.0f;
  for (int64_t k0 = 8 * (int64_t)threadIdx.x; k0 < a.k; k0 += 8 * 256) {
    const float4 v0 = *reinterpret_cast<const float4 *>(src + k0);
    const float4 v1 = *reinterpret_cast<const float4 *>(src + k0 + 4);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))));
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)), fmaxf(fabsf(v1.z), fabsf(v1.w))));
  }
  const int e = f16_row_exponent(block_max_256(amax));
  if (threadIdx.x == 0) a.exp_out[row] = e;
  uint16_t *dst = a.out + row * 2 * a.k;
  for (int64_t k0 = 8 * (int64_t)threadIdx.x; k0 < a.k; k0 += 8 * 256) {
    const float4 v0 = *reinterpret_cast<const float4 *>(src + k0);
    const float4 v1 = *reinterpret_cast<const float4 *>(src + k0 + 4);
    const float w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    f16x8 h, l;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      _Float16 hu, lu;
      split_f16(w[u], e, hu, lu);
      h[u] = hu;
      l[u] = lu;
    }
    *reinterpret_cast<f16x8 *>(dst + k0) = h;
    *reinterpret_cast<f16x8 *>(dst + a.k + k0) = l;
  }
}

// one wavefront per row of x: the scale exponent of the row
__global__ __launch_bounds__(256) void row_exponents_kernel(const float *x, int64_t m, int64_t k, int64_t lda,
                                                            int32_t *out) {
  const int64_t row = 4 * (int64_t)blockIdx.x + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= m) return;
  const float *p = x + row * lda;
  float amax = 0.0f;
  // 16 loads of 16 bytes in flight per lane (a 4096-wide row in one round)
  for (int64_t c0 = 4 * lane; c0 < k; c0 += 256 * 16) {
    float4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      v[u] = c0 + 256 * u < k ? *reinterpret_cast<const float4 *>(p + c0 + 256 * u) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < 16; ++u)
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w))));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (lane == 0) out[row] = f16_row_exponent(amax);
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

  // L2 prefetch of a later stage's x lines (as in gemm_x6_kernel): loading
  // lane (lw, l) touches row 64 lw + l of a full row tile. A row's stage is
  // KPS bf16 values; with 64 of them two stages share a 128-byte line, which
  // is then touched on even stages only.
  static_assert(KPS * 2 == 64 || KPS * 2 == 128, "x bytes per row and stage");
  static_assert(BM == 64 * NL, "one tile row per loading lane");
  constexpr int PF_EVERY = 128 / (KPS * 2);
  const bool full_tile = a_rows == BM;
  __shared__ __attribute__((aligned(16))) uint32_t pf_sink[NL][64];
  const uint32_t pf_voff = (uint32_t)((64 * lw + lane) * g.lda * 2);
  auto prefetch = [&](int kt) {
    buffer_load_lds(a_rsrc, (lds_u32 *)(&pf_sink[lw][0]), 4, (int32_t)pf_voff, (int32_t)(kt * KPS * 2), 0, 0);
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
    wait_vm0_seen();
  }
  phase_barrier();
  if (!loader) phase_barrier();  // group 4..7 runs one phase behind
  for (int kt = 0; kt < kt_count; ++kt) {
    const int st = kt & 1;
    // the stage load may go out before this phase's LDS reads (as in
    // gemm_x6_kernel); only the pooling instance does so, the others would
    // get a wait for every load in flight before their first LDS read
    constexpr bool kLoadFirst = POOL;
    if (!kLoadFirst) reads(st);
    if (loader && kt + 1 < kt_count) issue(kt + 1, st ^ 1);
    const int pf_stage = kt + 1 + kXPrefetch;
    const bool pf = kXPrefetch > 0 && loader && full_tile && pf_stage < kt_count && pf_stage % PF_EVERY == 0;
    if (pf) prefetch(pf_stage);
    if (kLoadFirst) reads(st);
    wait_lgkm0();  // this stage's reads are done before its buffer can be reloaded
    phase_barrier();
    mfmas();
    if (loader) {  // the next stage has landed before this group reads it
      if (pf) wait_vm1_seen();  // (the line touch may still be in flight)
      else wait_vm0_seen();
    }
    phase_barrier();
  }
  if (loader) phase_barrier();  // the same number of barriers for every wavefront

  if constexpr (POOL) {
    pool_epilogue<WM, WN, true>(g, acc, smem, m0, 64 * nt, wm, wn, lane);
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

// F16: the same kernel on the f16 matrix cores (v_mfma_f32_16x16x32_f16)
// with the two-part f16 weights: each row fragment's x row brings its scale
// exponent (g.xexp), the split gives xh, xl (split8_f16), and the multiply
// phase sums xh wh, xh wl, xl wh (the left-out xl wl is at most 2^-22 |x w|
// of the scaled values); the epilogue scales every sum back by
// 2^-(xexp + wexp), exactly, before the bias and the pooling. With two
// weight parts the kernel also runs 256 x 256 tiles of eight 64 x 128
// wavefronts (twice the matrix-core work per LDS stage and per barrier; the
// x split is shared by twice the MFMAs).
// y - h for h one half of a packed f16 pair: one fused multiply-add with the
// f16 operand taken as is (-h * 1 + y, exact), in place of converting h back
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float residual_lo(uint32_t hpair, float y) {
  float r;
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hpair), "v"(y));
  return r;
}
__device__ __forceinline__ float residual_hi(uint32_t hpair, float y) {
  float r;
  asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(hpair), "v"(y));
  return r;
}

__device__ __forceinline__ void split8_f16(const f4 lo4, const f4 hi4, int e, f16x8 &h, f16x8 &l) {
  const float v[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float y0 = __builtin_amdgcn_ldexpf(v[2 * u], e), y1 = __builtin_amdgcn_ldexpf(v[2 * u + 1], e);
    hw[u] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{y0, y1}), f16x2));
    const float r0 = residual_lo(hw[u], y0), r1 = residual_hi(hw[u], y1);
    lw[u] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{r0, r1}), f16x2));
  }
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  h = __builtin_bit_cast(f16x8, (u4{hw[0], hw[1], hw[2], hw[3]}));
  l = __builtin_bit_cast(f16x8, (u4{lw[0], lw[1], lw[2], lw[3]}));
}

template <bool POOL, bool F16, int BN = 128, int WN = 64>
__global__ __launch_bounds__(512, 1) void gemm_x6_kernel(GemmArgs g) {
  constexpr int BM = 256, WM = 64, BK = kBK3;
  constexpr int WAVES_N = BN / WN;  // 2
  static_assert(WAVES_N == 2 && (BN == 128 || (F16 && BN == 256)), "tile");
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int BRB = BN / 16;
  constexpr int NL = 4;
  constexpr int NP = F16 ? 2 : 3;                   // weight parts
  constexpr int A_INS = BM / 8 / NL, B_INS = NP * BRB / NL;  // x: 8 rows of 32 floats per load
  constexpr int STAGE_FLOATS = 2 * (BM * BK + NP * BN * BK / 2);
  constexpr int SMEM_FLOATS = POOL && kPoolXFloats > STAGE_FLOATS ? kPoolXFloats : STAGE_FLOATS;
  static_assert(SMEM_FLOATS * 4 <= 160 * 1024, "LDS");
  typedef typename std::conditional<F16, f16x8, bf16x8>::type v8;
  __shared__ __attribute__((aligned(16))) float smem[SMEM_FLOATS];
  float(*As)[BM * BK] = reinterpret_cast<float(*)[BM * BK]>(smem);
  uint16_t(*Bs)[NP][BN * BK] = reinterpret_cast<uint16_t(*)[NP][BN * BK]>(smem + 2 * BM * BK);

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
  // (l % 8) ^ ((l / 8) & 7); weights as gemm_mc_kernel (rows of NP k).
  const int64_t RS = NP * g.k;
  const int64_t a_rows = (g.m - m0 < BM) ? (g.m - m0) : BM;
  const i32x4 a_rsrc = uniform_rsrc(make_rsrc(g.a + m0 * g.lda, (uint32_t)(a_rows * g.lda * 4)));
  const i32x4 b_rsrc = uniform_rsrc(make_rsrc(g.bsplit + n_glob * RS, (uint32_t)(BN * RS * 2)));
  const int xr = lane >> 3, xq = (lane & 7) ^ (xr & 7);
  // a full row tile: one lane offset, the row step of each load in the
  // scalar offset; the ragged last tile clamps each load's row instead
  // (rows past m read a valid row and are never stored)
  const bool full_tile = a_rows == BM;
  const uint32_t a_voff0 = (uint32_t)(((int64_t)(8 * lw * A_INS) + xr) * g.lda * 4 + 16 * xq);
  const int lr = lane >> 2, lq = (lane & 3) ^ ((lr >> 1) & 3);
  const uint32_t b_voff = (uint32_t)((lr * RS + 8 * lq) * 2);
  auto issue = [&](int kt, int st) {
    if (full_tile) {
#pragma unroll
      for (int u = 0; u < A_INS; ++u)
        buffer_load_lds(a_rsrc, (lds_u32 *)(&As[st][256 * (lw * A_INS + u)]), 16, (int32_t)a_voff0,
                        (int32_t)(kt * BK * 4 + u * 8 * g.lda * 4), 0, 0);
    } else {
#pragma unroll
      for (int u = 0; u < A_INS; ++u) {
        int64_t r = 8 * (lw * A_INS + u) + xr;
        if (r >= a_rows) r = a_rows - 1;
        buffer_load_lds(a_rsrc, (lds_u32 *)(&As[st][256 * (lw * A_INS + u)]), 16, (int32_t)((r * g.lda + 4 * xq) * 4),
                        (int32_t)(kt * BK * 4), 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < B_INS; ++u) {
      const int q = lw * B_INS + u, p = q / BRB, rb = q % BRB;
      buffer_load_lds(b_rsrc, (lds_u32 *)(&Bs[st][p][512 * rb]), 16, (int32_t)b_voff,
                      (int32_t)((uint32_t)(kt * BK * 2) + (uint32_t)((rb * 16 * RS + p * g.k) * 2)), 0, 0);
    }
  };

  // L2 prefetch of a later stage's x lines: loading lane (lw, l) touches row
  // 64 lw + l (full row tiles only); the 4 bytes land in a scratch LDS row
  __shared__ __attribute__((aligned(16))) uint32_t pf_sink[NL][64];
  const uint32_t pf_voff = (uint32_t)((64 * lw + lane) * g.lda * 4);
  auto prefetch = [&](int kt) {
    buffer_load_lds(a_rsrc, (lds_u32 *)(&pf_sink[lw][0]), 4, (int32_t)pf_voff, (int32_t)(kt * BK * 4), 0, 0);
  };

  f4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  const int row_in = lane & 15, slot = lane >> 4;
  // F16: the scale exponent of the x row each row fragment reads
  int xe[FM];
  if constexpr (F16) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      int64_t r = wm * WM + 16 * i + row_in;
      if (r >= a_rows) r = a_rows - 1;
      xe[i] = g.xexp[m0 + r];
    }
  }
  // the read phase keeps x as f32 (8 values per row fragment) and splits row
  // fragment 0; the multiply phase splits row fragment i + 1 while row
  // fragment i's MFMAs run
  f4 xf[FM][2];
  v8 fa[2][NP], fb[NP][FN];
  auto split = [&](int i, v8 (&parts)[NP]) {
    if constexpr (F16) split8_f16(xf[i][0], xf[i][1], xe[i], parts[0], parts[1]);
    else split8(xf[i][0], xf[i][1], parts[0], parts[1], parts[2]);
  };
  auto reads = [&](int st) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WM + 16 * i + row_in;
      xf[i][0] = *reinterpret_cast<const f4 *>(&As[st][r * BK + 4 * ((2 * slot) ^ (r & 7))]);
      xf[i][1] = *reinterpret_cast<const f4 *>(&As[st][r * BK + 4 * ((2 * slot + 1) ^ (r & 7))]);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WN + 16 * j + row_in;
        fb[p][j] = *reinterpret_cast<const v8 *>(&Bs[st][p][r * BK + 8 * (slot ^ ((r >> 1) & 3))]);
      }
    // row fragment 0 split here, so the multiply phase opens with MFMAs
    split(0, fa[0]);
  };
  // per row fragment, the part products in the order xh wh, xh wm, xm wh,
  // xh wl, xm wm, xl wh (F16: xh wh, xh wl, xl wh); every output sums them in
  // that order
  auto mfmas = [&]() {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int cur = i & 1;
      if (i + 1 < FM) split(i + 1, fa[cur ^ 1]);
      if constexpr (F16) {
        constexpr int XP[3] = {0, 0, 1}, WP[3] = {0, 1, 0};
#pragma unroll
        for (int q = 0; q < 3; ++q)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[cur][XP[q]], fb[WP[q]][j], acc[i][j], 0, 0, 0);
        // the next fragment's split (24 vector instructions) interleaved one
        // by one with this fragment's MFMAs
#pragma unroll
        for (int q = 0; q < 3 * FN; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i + 1 < FM && q < 24) __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
        }
      } else {
        constexpr int XP[6] = {0, 0, 1, 0, 1, 2}, WP[6] = {0, 1, 0, 2, 1, 0};
#pragma unroll
        for (int q = 0; q < 6; ++q)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[cur][XP[q]], fb[WP[q]][j], acc[i][j], 0, 0, 0);
      }
    }
  };

  if (loader) issue(0, 0);
  // every wavefront drains its loads here (the first stage, the exponents),
  // so that no wait for them lands inside the loop
  wait_vm0_seen();
  if (kXPrefetch > 0 && loader && full_tile) {
    for (int s = 2; s <= kXPrefetch && s < kt_count; ++s) prefetch(s);
  }
  phase_barrier();
  if (!loader) phase_barrier();  // group 4..7 runs one phase behind
  for (int kt = 0; kt < kt_count; ++kt) {
    const int st = kt & 1;
    // The stage load may go out before this phase's LDS reads: its buffer
    // was last read before the previous phase barrier (the other group's
    // reads of it end before the barrier that ends this group's multiply
    // phase). The f16 256 x 256 instances do so; in the others the compiler
    // then waits for every load in flight before the first LDS read (it
    // cannot tell the stage buffers apart), so those read first.
    constexpr bool kLoadFirst = F16 && BN == 256;
    if (!kLoadFirst) reads(st);
    if (loader && kt + 1 < kt_count) issue(kt + 1, st ^ 1);
    // the line touch of stage kt + 1 + kXPrefetch goes after the stage load,
    // so that waiting for all loads but the last one covers the stage
    const bool pf = kXPrefetch > 0 && loader && full_tile && kt + 1 + kXPrefetch < kt_count;
    if (pf) prefetch(kt + 1 + kXPrefetch);
    if (kLoadFirst) reads(st);
    wait_lgkm0();
    phase_barrier();
    mfmas();
    if (loader) {
      if (pf) wait_vm1_seen();  // the stage load has landed, the line touch may still be in flight
      else wait_vm0_seen();
    }
    phase_barrier();
  }
  if (loader) phase_barrier();  // the same number of barriers for every wavefront

  if constexpr (F16) {
    // back from the scaled rows: output (row, column) times 2^-(xexp + wexp)
    int we[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) we[j] = g.wexp[n_glob + wn * WN + 16 * j + row_in];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int64_t rr = wm * WM + 16 * i + 4 * slot + r;
        if (rr >= a_rows) rr = a_rows - 1;
        const int e = g.xexp[m0 + rr];
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j][r] = __builtin_amdgcn_ldexpf(acc[i][j][r], -(e + we[j]));
      }
  }
  if constexpr (POOL) {
    pool_epilogue<WM, WN>(g, acc, smem, m0, (BN / 4) * nt, wm, wn, lane);
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
      (a.pool_hd && (a.pool_tile != 256 && a.pool_tile != 128)) || (a.pool_hd && a.pool_hd % (a.pool_tile / 4) != 0) ||
      (a.pool_hd && (a.pool_wn != 64 && a.pool_wn != 128)) || (a.pool_hd && a.pool_tile % a.pool_wn != 0))
    return hipErrorInvalidValue;
  if (a.f16) {
    if (!a.exp_out) return hipErrorInvalidValue;
    hipLaunchKernelGGL(gemm::split_weights_f16_kernel, dim3((uint32_t)(2 * a.n_half)), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
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

namespace {
// shapes of the f32-x kernels (plain: n_half % 128 == 0; pooling: 32-feature
// column tiles, 4-token blocks aligned with the flattened rows)
bool x6_shape_ok(const GemmArgs &g, int parts, bool pool, int bn) {
  if (g.lda < g.k || g.k % gemm::kBK3 != 0 || (int64_t)256 * g.lda * 4 > INT32_MAX ||
      (int64_t)bn * parts * g.k * 2 > INT32_MAX)
    return false;
  if (pool)
    return g.pool_hd % (bn / 4) == 0 && g.n_half == 2 * (int64_t)g.pool_hd && g.ldc == 2 * g.pool_hd &&
           g.m == g.pool_batch * g.pool_seqlen && (g.pool_batch == 1 || g.pool_seqlen % 4 == 0) && g.pooled;
  return g.n_half % bn == 0 &&
         (!g.bias1 || (g.bias_seqlen >= 1 && g.bias_ratio >= 1 && (g.bias_ratio & (g.bias_ratio - 1)) == 0));
}

template <bool POOL, bool F16, int BN = 128, int WN = 64>
hipError_t launch_x6(const GemmArgs &g, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  if (!x6_shape_ok(g, F16 ? 2 : 3, POOL, BN) || (F16 && (!g.xexp || !g.wexp))) return hipErrorInvalidValue;
  const int64_t m_tiles = (g.m + 255) / 256;
  const int64_t n_tiles = POOL ? g.pool_hd / (BN / 4) : 2 * g.n_half / BN;
  hipLaunchKernelGGL((gemm::gemm_x6_kernel<POOL, F16, BN, WN>), dim3((uint32_t)(m_tiles * n_tiles)), dim3(512), 0,
                     stream, g);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_x6(const GemmArgs &g, hipStream_t stream) { return launch_x6<false, false>(g, stream); }
hipError_t launch_gemm_x6_pool(const GemmArgs &g, hipStream_t stream) { return launch_x6<true, false>(g, stream); }
// f16 parts: 256 x 256 tiles of 64 x 128 wavefronts where the columns allow
hipError_t launch_gemm_h3(const GemmArgs &g, hipStream_t stream) {
  if (g.n_half % 256 == 0) return launch_x6<false, true, 256, 128>(g, stream);
  return launch_x6<false, true>(g, stream);
}
hipError_t launch_gemm_h3_pool(const GemmArgs &g, hipStream_t stream) { return launch_x6<true, true, 256, 128>(g, stream); }

hipError_t launch_row_exponents(const float *x, int64_t m, int64_t k, int64_t lda, int32_t *out,
                                hipStream_t stream) {
  if (m <= 0) return hipSuccess;
  if (k <= 0 || k % 4 != 0 || lda < k || lda % 4 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm::row_exponents_kernel, dim3((uint32_t)((m + 3) / 4)), dim3(256), 0, stream, x, m, k, lda,
                     out);
  return hipGetLastError();
}

}  // namespace kvc
