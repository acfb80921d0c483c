// Fused pooling kernels of the compressor (gfx950): positional bias, the
// candidate window, per-feature softmax pooling, bf16 rounding, RMSNorm and
// the fp4 round trip of each compressed entry, plus the state hand-off kernels
// and the standalone fp4 quantiser.
//
// Pooling: "DeepSeek V4.1 . Pool token pairs", pooling formula and Compressor
// listing (forward). Overlap at ratio 4: "Compressed Sparse Attention . ratio
// m = 4", Why one output uses eight candidates. Precision: "Module compress",
// Precision paragraph. fp4: "Module compress", Functions,
// fp4_quant_e4m3_inplace / to_e2m1_rne.
//
// Memory-bound work: every kernel streams f32 projection rows with 16-byte
// (or 8-byte) coalesced loads, one wavefront per 64 x VEC features, and keeps
// all per-entry arithmetic in registers.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {
namespace {

// Round-robin dispatch puts consecutive workgroups on different XCDs; remap
// so that each XCD works on one contiguous range of the sequence, keeping
// neighbouring entries (which share a block of rows at ratio 4) in one L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t n) {
  const uint32_t q = n / 8, r = n % 8, x = id % 8, local = id / 8;
  return (x < r) ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

// Lane layout of one entry's HD features across a wavefront: chunks of QV
// consecutive features (one 4*QV-byte access each), H = HD / (64*QV) chunks
// per lane; chunk h of lane l holds features h*64*QV + l*QV + [0, QV). Every
// load instruction of a wavefront then covers one contiguous span of 64*QV
// floats, and a block of 16 features (one fp4 scale) spans 16/QV lanes.
template <int HD>
struct Lanes {
  static constexpr int VEC = HD / kWave;
  static constexpr int QV = VEC >= 4 ? 4 : VEC;
  static constexpr int H = VEC / QV;
  static_assert(QV == 2 || QV == 4, "head_dim must be 128 or a multiple of 256");
  __device__ static int feature(int lane, int h) { return h * kWave * QV + lane * QV; }
};

template <int QV>
__device__ __forceinline__ void load_q(const float *p, float *d) {
  if constexpr (QV == 4) {
    const float4 t = *reinterpret_cast<const float4 *>(p);
    d[0] = t.x; d[1] = t.y; d[2] = t.z; d[3] = t.w;
  } else {
    static_assert(QV == 2, "QV must be 2 or 4");
    const float2 t = *reinterpret_cast<const float2 *>(p);
    d[0] = t.x; d[1] = t.y;
  }
}

// The same load marked non-temporal (streamed: each projection value is read
// once per launch, so its line need not displace data that is reused). On
// gfx950 this lifts the pooling kernels from about 0.68 to 0.77 of HBM peak.
template <int QV>
__device__ __forceinline__ void load_q_stream(const float *p, float *d) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  if constexpr (QV == 4) {
    const f4 t = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(p));
    d[0] = t.x; d[1] = t.y; d[2] = t.z; d[3] = t.w;
  } else {
    static_assert(QV == 2, "QV must be 2 or 4");
    const f2 t = __builtin_nontemporal_load(reinterpret_cast<const f2 *>(p));
    d[0] = t.x; d[1] = t.y;
  }
}

template <int QV>
__device__ __forceinline__ void store_q(float *p, const float *d) {
  if constexpr (QV == 4) *reinterpret_cast<float4 *>(p) = make_float4(d[0], d[1], d[2], d[3]);
  else *reinterpret_cast<float2 *>(p) = make_float2(d[0], d[1]);
}

// QV bf16 patterns (low 16 bits of each word) as one store
template <int QV>
__device__ __forceinline__ void store_bf16_q(uint16_t *p, const uint32_t *b) {
  if constexpr (QV == 4) *reinterpret_cast<uint2 *>(p) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
  else *reinterpret_cast<uint32_t *>(p) = b[0] | (b[1] << 16);
}

// One token row's VEC features of this lane (layout Lanes<HD>), `base` at
// the row's first feature.
template <int HD>
__device__ __forceinline__ void load_row(const float *base, int lane, float (&d)[HD / kWave]) {
  using L = Lanes<HD>;
#pragma unroll
  for (int h = 0; h < L::H; ++h) load_q<L::QV>(base + L::feature(lane, h), d + h * L::QV);
}

template <int HD>
__device__ __forceinline__ void load_row_stream(const float *base, int lane, float (&d)[HD / kWave]) {
  using L = Lanes<HD>;
#pragma unroll
  for (int h = 0; h < L::H; ++h) load_q_stream<L::QV>(base + L::feature(lane, h), d + h * L::QV);
}

template <int HD>
__device__ __forceinline__ void store_row(float *base, int lane, const float (&d)[HD / kWave]) {
  using L = Lanes<HD>;
#pragma unroll
  for (int h = 0; h < L::H; ++h) store_q<L::QV>(base + L::feature(lane, h), d + h * L::QV);
}

// Per-entry epilogue of one wavefront holding the entry's pooled features
// (layout Lanes<HD>): optional f32 store, bf16 round, RMSNorm over the entry
// (wave reduction), bf16 latent, optional RoPE of the rotary slice (table row
// rope_row; a lane's rotary pairs lie inside its own chunks), and the fp4
// codes / scales / dequantised values of the cached (rotated, with RoPE) entry.
template <int HD>
__device__ __forceinline__ void finish_entry(const float (&p)[HD / kWave], const PoolArgs &a, int64_t out_row,
                                             int64_t rope_row, int lane) {
  using L = Lanes<HD>;
  constexpr int VEC = L::VEC, QV = L::QV;
  if (a.pooled) store_row<HD>(a.pooled + out_row * HD, lane, p);
  float u[VEC];
  float ss = 0.0f;
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    u[v] = bf16_val(bf16_rne(p[v]));
    ss = __builtin_fmaf(u[v], u[v], ss);
  }
  ss = wave_sum(ss);
  const float r = __builtin_amdgcn_rsqf(ss * (1.0f / HD) + a.eps);
  float y[VEC];
  uint32_t yb[VEC];
#pragma unroll
  for (int h = 0; h < L::H; ++h)
#pragma unroll
    for (int q = 0; q < QV; ++q) {
      const int v = h * QV + q;
      float t = u[v] * r;
      if (a.norm_w) t *= a.norm_w[L::feature(lane, h) + q];
      yb[v] = bf16_rne(t);
      y[v] = bf16_val(yb[v]);
    }
  if (a.latent) {
#pragma unroll
    for (int h = 0; h < L::H; ++h) store_bf16_q<QV>(a.latent + out_row * HD + L::feature(lane, h), yb + h * QV);
  }
  if (a.rope_cs) {
    const float *row = a.rope_cs + rope_row * a.rope_dim;
    const int start = HD - a.rope_dim;
#pragma unroll
    for (int h = 0; h < L::H; ++h)
#pragma unroll
      for (int q = 0; q < QV; q += 2) {
        const int f = L::feature(lane, h) + q, v = h * QV + q;
        if (f >= start) {
          const float2 cs = *reinterpret_cast<const float2 *>(row + (f - start));
          rope_pair(y[v], y[v + 1], cs.x, cs.y, yb[v], yb[v + 1]);
          y[v] = bf16_val(yb[v]);
          y[v + 1] = bf16_val(yb[v + 1]);
        }
      }
    if (a.rotated) {
#pragma unroll
      for (int h = 0; h < L::H; ++h) store_bf16_q<QV>(a.rotated + out_row * HD + L::feature(lane, h), yb + h * QV);
    }
  }
  // the fp4 forms, each instance computing the dequantised values only when
  // they are stored (the flags are uniform across the launch)
  auto fp4_out = [&](auto e8m0_tag, auto deq_tag) {
    constexpr bool E8 = decltype(e8m0_tag)::value, DQ = decltype(deq_tag)::value;
    constexpr int blk = E8 ? 32 : 16;
#pragma unroll
    for (int h = 0; h < L::H; ++h) {
      const int f = L::feature(lane, h);
      float yq[QV];
#pragma unroll
      for (int q = 0; q < QV; ++q) yq[q] = y[h * QV + q];
      uint32_t packed, scode, deq[QV];
      if constexpr (E8) fp4_block_e8m0<QV, DQ>(yq, packed, scode, deq);
      else fp4_block<QV, DQ>(yq, packed, scode, deq);
      if (a.codes) {
        uint8_t *c = a.codes + out_row * (HD / 2) + f / 2;
        if constexpr (QV == 4) *reinterpret_cast<uint16_t *>(c) = (uint16_t)packed;
        else *c = (uint8_t)packed;
      }
      if (a.scales && (f % blk) == 0) a.scales[out_row * (HD / blk) + f / blk] = (uint8_t)scode;
      if constexpr (DQ) store_bf16_q<QV>(a.deq + out_row * HD + f, deq);
    }
  };
  using yes = std::true_type;
  using no = std::false_type;
  if (a.deq) {
    if (a.e8m0) fp4_out(yes{}, yes{});
    else fp4_out(no{}, yes{});
  } else if (a.codes || a.scales) {
    if (a.e8m0) fp4_out(yes{}, no{});
    else fp4_out(no{}, no{});
  }
}

// The candidates of one entry of a small group (ratio 2, ratio 4
// overlapped) in this lane's features (layout Lanes<HD>), from kv/score
// planes holding the token rows of batch row b. Ratio 4: entry j pools rows
// 4(j-1)..4j-1 of branch B (columns [HD, 2HD)) then rows 4j..4j+3 of branch
// A (columns [0, HD)); entry 0's previous branch is kv 0 / score -inf. The
// entry loads exactly its own candidates.
template <int HD, int R, bool OV>
struct Candidates {
  static constexpr int VEC = HD / kWave;
  static constexpr int NC = OV ? 2 * R : R;
  static constexpr int C0 = OV ? R : 0;  // the current block's first candidate
  float k[NC][VEC], s[NC][VEC];          // in pooling order: [previous B,] current rows
};

template <int HD, int R, bool OV>
__device__ __forceinline__ void load_candidates(const PoolArgs &a, int64_t b, int64_t j, int lane,
                                                Candidates<HD, R, OV> &c) {
  constexpr int VEC = HD / kWave, C0 = Candidates<HD, R, OV>::C0;
  const float *KV = a.kv + b * a.batch_stride;
  const float *SC = a.sc + b * a.batch_stride;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int64_t row = (int64_t)R * j + i;
    load_row_stream<HD>(KV + row * a.row_stride, lane, c.k[C0 + i]);
    load_row_stream<HD>(SC + row * a.row_stride, lane, c.s[C0 + i]);
  }
  if constexpr (OV) {
    if (j > 0) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int64_t row = (int64_t)R * (j - 1) + i;
        load_row_stream<HD>(KV + row * a.row_stride + HD, lane, c.k[i]);
        load_row_stream<HD>(SC + row * a.row_stride + HD, lane, c.s[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int v = 0; v < VEC; ++v) { c.k[i][v] = 0.0f; c.s[i][v] = -INFINITY; }
    }
  }
  if (a.ape) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float bias[VEC];
      load_row<HD>(a.ape + (int64_t)i * a.row_stride, lane, bias);
#pragma unroll
      for (int v = 0; v < VEC; ++v) c.s[C0 + i][v] += bias[v];
      if constexpr (OV) {
        load_row<HD>(a.ape + (int64_t)i * a.row_stride + HD, lane, bias);
#pragma unroll
        for (int v = 0; v < VEC; ++v) c.s[i][v] += bias[v];  // -inf padding stays -inf
      }
    }
  }
}

// The pooled entry (output e of batch row b) from its candidates: softmax
// pooling, then the per-entry epilogue.
template <int HD, int R, bool OV>
__device__ __forceinline__ void pool_candidates(const PoolArgs &a, int64_t b, int64_t e, int lane,
                                                const Candidates<HD, R, OV> &c) {
  constexpr int VEC = HD / kWave;
  float p[VEC];
  softmax_pool<Candidates<HD, R, OV>::NC, VEC>(c.k, c.s, p);
  finish_entry<HD>(p, a, b * a.out_batch_stride + e, a.rope_row0 + e, lane);
}

// One entry of a small group by one wavefront (features laid out as
// Lanes<HD>). With shift_kv set (decode), the block just pooled is then
// copied to the previous-block rows; the lane only touches features it
// alone reads.
template <int HD, int R, bool OV>
__device__ __forceinline__ void small_entry(const PoolArgs &a, int64_t b, int64_t e, int lane) {
  constexpr int VEC = HD / kWave, C0 = Candidates<HD, R, OV>::C0;
  const int64_t j = a.first_entry + e;
  Candidates<HD, R, OV> c;
  load_candidates<HD, R, OV>(a, b, j, lane, c);
  pool_candidates<HD, R, OV>(a, b, e, lane, c);

  if constexpr (OV) {
    if (a.shift_kv) {
      const float *KV = a.kv + b * a.batch_stride;
      const float *SC = a.sc + b * a.batch_stride;
      float *SK = a.shift_kv + b * a.batch_stride;
      float *SS = a.shift_sc + b * a.batch_stride;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int64_t row = (int64_t)R * j + i;
        float bk[VEC], bs[VEC];
        load_row<HD>(KV + row * a.row_stride + HD, lane, bk);
        load_row<HD>(SC + row * a.row_stride + HD, lane, bs);
        const int64_t dst = (int64_t)R * (j - 1) + i;
        store_row<HD>(SK + dst * a.row_stride, lane, c.k[C0 + i]);
        store_row<HD>(SS + dst * a.row_stride, lane, c.s[C0 + i]);
        store_row<HD>(SK + dst * a.row_stride + HD, lane, bk);
        store_row<HD>(SS + dst * a.row_stride + HD, lane, bs);
      }
    }
  }
}

// Small groups (ratio 2, ratio 4 overlapped): one wavefront walks a run of
// consecutive entries of one batch row. Every projection value is read once
// over the whole launch and nothing is carried from one entry to the next.
template <int HD, int R, bool OV>
__global__ __launch_bounds__(256) void pool_small_kernel(PoolArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * 4 + (threadIdx.x >> 6);
  const int64_t runs = (a.groups + a.entries_per_wave - 1) / a.entries_per_wave;
  const int64_t b = wave / runs;
  if (b >= a.batch) return;
  const int64_t run = wave - b * runs;
  const int64_t e_begin = run * a.entries_per_wave;
  const int64_t e_end = min(e_begin + (int64_t)a.entries_per_wave, a.groups);
  for (int64_t e = e_begin; e < e_end; ++e) small_entry<HD, R, OV>(a, b, e, lane);
}

// Decode at ratio 4, a group just completed: the entry of each batch row
// (workgroup b) from the state window, and the move of the block into the
// previous-block rows (rows R..2R-1 to 0..R-1, both halves, both planes).
// Wavefront 0 loads the candidates, wavefront 1 the rows to move; once both
// have their data (the barrier), wavefront 0 pools and wavefront 1 stores,
// so the move's round trip overlaps the pooling instead of following it.
// The state's scores already hold the bias (a.ape is null). Same bits as
// small_entry with shift_kv.
template <int HD, int R>
__global__ __launch_bounds__(128) void decode_emit_kernel(PoolArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t b = blockIdx.x;
  const int64_t j = a.first_entry;
  // wavefront 0: the candidates; wavefront 1: the 2 R half rows to move, in
  // the same registers (slot 2 i + h: row R j + i, half h)
  Candidates<HD, R, true> c;
  static_assert(Candidates<HD, R, true>::NC == 2 * R, "one slot per half row");
  if (wave == 0) {
    load_candidates<HD, R, true>(a, b, j, lane, c);
  } else {
    const float *KV = a.kv + b * a.batch_stride;
    const float *SC = a.sc + b * a.batch_stride;
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t off = ((int64_t)R * j + i) * a.row_stride + h * HD;
        load_row<HD>(KV + off, lane, c.k[2 * i + h]);
        load_row<HD>(SC + off, lane, c.s[2 * i + h]);
      }
  }
  __builtin_amdgcn_s_waitcnt(0);  // every load of this wavefront has returned
  __syncthreads();                // and the other wavefront's
  if (wave == 0) {
    pool_candidates<HD, R, true>(a, b, 0, lane, c);
  } else {
    float *SK = a.shift_kv + b * a.batch_stride;
    float *SS = a.shift_sc + b * a.batch_stride;
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t off = ((int64_t)R * (j - 1) + i) * a.row_stride + h * HD;
        store_row<HD>(SK + off, lane, c.k[2 * i + h]);
        store_row<HD>(SS + off, lane, c.s[2 * i + h]);
      }
  }
}

// Ratio 1: every row of f32 projections is one entry; one wavefront runs the
// per-entry epilogue of one row (the same code as the pooled entries).
template <int HD>
__global__ __launch_bounds__(256) void rows_finish_kernel(PoolArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t e = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= a.groups) return;
  float p[HD / kWave];
  load_row<HD>(a.kv + e * a.row_stride, lane, p);
  // rows are [batch][entries]: the RoPE row is the entry's index in its batch row
  finish_entry<HD>(p, a, e, a.rope_row0 + e % a.out_batch_stride, lane);
}

// Ratio 4 after the pooling GEMM: the first entry of every row tile t >= 1
// (4-token block 64 t of the flattened rows) whose previous block belongs to
// the row tile above, pooled by the small-group code from the plane rows the
// GEMM wrote; only p.pooled is written.
template <int HD>
__global__ __launch_bounds__(256) void pool_boundary_kernel(PoolArgs a, int64_t row_tiles, int64_t seqlen) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = 1 + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= row_tiles) return;
  const int64_t gf = 64 * t;
  const int64_t b = a.batch == 1 ? 0 : gf / (seqlen / 4);
  const int64_t j = a.batch == 1 ? gf : gf - b * (seqlen / 4);
  if (b >= a.batch || j == 0 || j >= a.groups) return;
  small_entry<HD, 4, true>(a, b, j, lane);
}

// Long groups (ratio 128). One workgroup of 512 threads per entry: thread t
// owns 4 features (fg = t % (HD/4)) and every RL-th row of the group
// (rl = t / (HD/4)), keeping a running max / sum / weighted sum per feature
// over chunks of CH rows. The RL partial states are merged in LDS by the
// first wavefront, which then runs the per-entry epilogue.
template <int HD, int R>
__global__ __launch_bounds__(512) void pool_long_kernel(PoolArgs a) {
  constexpr int FG = HD / 4;        // feature groups of 4
  constexpr int RL = 512 / FG;      // row lanes
  constexpr int ROWS = R / RL;      // rows per row lane
  constexpr int CH = 8;             // rows per chunk
  static_assert(ROWS % CH == 0, "rows per row lane must be a multiple of the chunk");
  constexpr int VEC = HD / kWave;   // features per lane in the epilogue
  using L = Lanes<HD>;
  __shared__ float s_m[RL][HD], s_l[RL][HD], s_acc[RL][HD];

  const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t b = id / a.groups;
  const int64_t e = id - b * a.groups;
  const int64_t j = a.first_entry + e;
  const int t = threadIdx.x;
  const int fg = t % FG, rl = t / FG;
  const float *KV = a.kv + b * a.batch_stride + (int64_t)R * j * a.row_stride + 4 * fg;
  const float *SC = a.sc + b * a.batch_stride + (int64_t)R * j * a.row_stride + 4 * fg;

  float m[4], l[4], acc[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) { m[v] = -INFINITY; l[v] = 0.0f; acc[v] = 0.0f; }
  for (int c = 0; c < ROWS / CH; ++c) {
    float k[CH][4], s[CH][4];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int row = (c * CH + i) * RL + rl;
      load_q_stream<4>(KV + (int64_t)row * a.row_stride, k[i]);
      load_q_stream<4>(SC + (int64_t)row * a.row_stride, s[i]);
    }
    if (a.ape) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int row = (c * CH + i) * RL + rl;
        float bias[4];
        load_q<4>(a.ape + (int64_t)row * a.row_stride + 4 * fg, bias);
#pragma unroll
        for (int v = 0; v < 4; ++v) s[i][v] += bias[v];
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float cm = m[v];
#pragma unroll
      for (int i = 0; i < CH; ++i) cm = __builtin_fmaxf(cm, s[i][v]);
      const float scale = __builtin_amdgcn_exp2f((m[v] - cm) * kLog2e);  // m = -inf -> 0
      float sl = 0.0f, sa = 0.0f;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const float ex = __builtin_amdgcn_exp2f((s[i][v] - cm) * kLog2e);
        sl += ex;
        sa = __builtin_fmaf(ex, k[i][v], sa);
      }
      l[v] = __builtin_fmaf(l[v], scale, sl);
      acc[v] = __builtin_fmaf(acc[v], scale, sa);
      m[v] = cm;
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    s_m[rl][4 * fg + v] = m[v];
    s_l[rl][4 * fg + v] = l[v];
    s_acc[rl][4 * fg + v] = acc[v];
  }
  __syncthreads();
  if (t >= kWave) return;
  const int lane = t;
  float p[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    const int f = L::feature(lane, v / L::QV) + v % L::QV;
    float mm = s_m[0][f];
#pragma unroll
    for (int r = 1; r < RL; ++r) mm = __builtin_fmaxf(mm, s_m[r][f]);
    float den = 0.0f, num = 0.0f;
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      const float w = __builtin_amdgcn_exp2f((s_m[r][f] - mm) * kLog2e);
      den = __builtin_fmaf(s_l[r][f], w, den);
      num = __builtin_fmaf(s_acc[r][f], w, num);
    }
    p[v] = num * __builtin_amdgcn_rcpf(den);
  }
  finish_entry<HD>(p, a, b * a.out_batch_stride + e, a.rope_row0 + e, lane);
}

__global__ __launch_bounds__(256) void state_store_kernel(StateStoreArgs s) {
  const int64_t c4 = s.proj / 4;
  const int64_t total = s.batch * s.state_rows * c4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int64_t c = (idx % c4) * 4;
  const int64_t row = (idx / c4) % s.state_rows;
  const int64_t b = idx / (c4 * s.state_rows);
  const int64_t n = s.seqlen / s.ratio, rem = s.seqlen - n * s.ratio;
  int64_t tok = -1;  // source token, or -1 for padding
  if (s.overlap) {
    if (row < s.ratio) {
      if (n > 0) tok = (n - 1) * s.ratio + row;
    } else {
      if (row - s.ratio >= rem) return;  // not part of the carry
      tok = n * s.ratio + (row - s.ratio);
    }
  } else {
    if (row >= rem) return;
    tok = n * s.ratio + row;
  }
  float4 k, g;
  if (tok < 0) {
    k = make_float4(0.f, 0.f, 0.f, 0.f);
    g = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  } else {
    const int64_t src = (b * s.seqlen + tok) * s.proj + c;
    k = *reinterpret_cast<const float4 *>(s.kv + src);
    g = *reinterpret_cast<const float4 *>(s.sc + src);
    if (s.ape) {
      const float4 bias = *reinterpret_cast<const float4 *>(s.ape + (tok % s.ratio) * s.proj + c);
      g.x += bias.x; g.y += bias.y; g.z += bias.z; g.w += bias.w;
    }
  }
  const int64_t dst = (b * s.state_rows + row) * s.proj + c;
  *reinterpret_cast<float4 *>(s.kv_state + dst) = k;
  *reinterpret_cast<float4 *>(s.sc_state + dst) = g;
}

// Decode step after the projection: one workgroup per batch row sums the
// split partial projections of the row's token in a fixed order, adds the
// slot's bias row and writes the state row (ratio 4 at position 0 also resets
// the previous-block rows). On a step that completes a group of a small
// ratio, the first wavefront then pools the state window with the same entry
// code as the prefill kernel (so decode and prefill compute identical entries
// from identical projections) and, at ratio 4, shifts the block.
template <int HD, int R, bool OV, bool POOL>
__global__ __launch_bounds__(256) void decode_finish_kernel(IngestArgs g, PoolArgs a) {
  const int64_t b = blockIdx.x;
  const int64_t plane = g.batch * g.proj;
  float *KS = g.kv_state + b * g.state_rows * g.proj;
  float *SS = g.sc_state + b * g.state_rows * g.proj;
  for (int64_t c = 4 * (int64_t)threadIdx.x; c < g.proj; c += 4 * (int64_t)blockDim.x) {
    float4 k = *reinterpret_cast<const float4 *>(g.part + b * g.proj + c);
    float4 s = *reinterpret_cast<const float4 *>(g.part + plane + b * g.proj + c);
    for (int sp = 1; sp < g.splits; ++sp) {  // fixed order: deterministic sums
      const float4 pk = *reinterpret_cast<const float4 *>(g.part + (2 * sp) * plane + b * g.proj + c);
      const float4 ps = *reinterpret_cast<const float4 *>(g.part + (2 * sp + 1) * plane + b * g.proj + c);
      k.x += pk.x; k.y += pk.y; k.z += pk.z; k.w += pk.w;
      s.x += ps.x; s.y += ps.y; s.z += ps.z; s.w += ps.w;
    }
    if (g.ape) {
      const float4 bias = *reinterpret_cast<const float4 *>(g.ape + (int64_t)g.slot * g.proj + c);
      s.x += bias.x; s.y += bias.y; s.z += bias.z; s.w += bias.w;
    }
    *reinterpret_cast<float4 *>(KS + (int64_t)g.state_row * g.proj + c) = k;
    *reinterpret_cast<float4 *>(SS + (int64_t)g.state_row * g.proj + c) = s;
    if (g.reset_prev) {
      for (int i = 0; i < g.ratio; ++i) {
        *reinterpret_cast<float4 *>(KS + (int64_t)i * g.proj + c) = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4 *>(SS + (int64_t)i * g.proj + c) =
            make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      }
    }
  }
  if constexpr (POOL) {
    __syncthreads();  // the state row written above is visible to the whole workgroup
    if (threadIdx.x < kWave) small_entry<HD, R, OV>(a, b, 0, threadIdx.x);
  }
}

// Standalone fp4 round trip: each thread owns 8 consecutive values (16 bytes)
// in each of kQuantChunks chunks 256 threads apart (all loads issued before
// any arithmetic, so that twice the bytes are in flight); two neighbouring
// lanes form a block of 16 (e4m3 scales), four a block of 32 (power-of-two
// scales). The value count is a multiple of the block, so all lanes of a
// block are in range together. Input and dequantised output are streamed
// with non-temporal accesses (each byte is touched once). In place (out ==
// in) is allowed: a thread reads its chunks before it writes them.
constexpr int kQuantChunks = 2;

template <bool E8M0, bool OUT>
__global__ __launch_bounds__(256) void fp4_quant_kernel(const uint16_t *in, int64_t n8, uint8_t *codes,
                                                        uint8_t *scales, uint16_t *out) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const int64_t base = (int64_t)blockIdx.x * (256 * kQuantChunks) + threadIdx.x;
  u4 raw[kQuantChunks];
#pragma unroll
  for (int u = 0; u < kQuantChunks; ++u) {
    const int64_t i = base + 256 * u;
    if (i < n8) raw[u] = __builtin_nontemporal_load(reinterpret_cast<const u4 *>(in + 8 * i));
  }
#pragma unroll
  for (int u = 0; u < kQuantChunks; ++u) {
    const int64_t i = base + 256 * u;
    if (i >= n8) break;
    float y[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      y[2 * q] = bf16_val(raw[u][q] & 0xffffu);
      y[2 * q + 1] = bf16_val(raw[u][q] >> 16);
    }
    uint32_t packed, scode, deq[8];
    if constexpr (E8M0) fp4_block_e8m0<8, OUT>(y, packed, scode, deq);
    else fp4_block<8, OUT>(y, packed, scode, deq);
    if (codes) *reinterpret_cast<uint32_t *>(codes + 4 * i) = packed;
    constexpr int per = E8M0 ? 4 : 2;  // threads per block
    if (scales && (i % per) == 0) scales[i / per] = (uint8_t)scode;
    if constexpr (OUT) {
      u4 t;
      t.x = deq[0] | (deq[1] << 16);
      t.y = deq[2] | (deq[3] << 16);
      t.z = deq[4] | (deq[5] << 16);
      t.w = deq[6] | (deq[7] << 16);
      __builtin_nontemporal_store(t, reinterpret_cast<u4 *>(out + 8 * i));
    }
  }
}

template <int HD, int R, bool OV>
hipError_t launch_small(const PoolArgs &p, hipStream_t stream) {
  const int64_t runs = (p.groups + p.entries_per_wave - 1) / p.entries_per_wave;
  const int64_t waves = p.batch * runs;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((pool_small_kernel<HD, R, OV>), dim3((uint32_t)blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_long(const PoolArgs &p, hipStream_t stream) {
  const int64_t blocks = p.batch * p.groups;
  hipLaunchKernelGGL((pool_long_kernel<HD, 128>), dim3((uint32_t)blocks), dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const PoolArgs &p, int ratio, int head_dim, hipStream_t stream) {
  if (p.batch <= 0 || p.groups <= 0) return hipSuccess;
  switch (ratio * 10000 + head_dim) {
    case 2 * 10000 + 512: return launch_small<512, 2, false>(p, stream);
    case 2 * 10000 + 128: return launch_small<128, 2, false>(p, stream);
    case 4 * 10000 + 512: return launch_small<512, 4, true>(p, stream);
    case 4 * 10000 + 128: return launch_small<128, 4, true>(p, stream);
    case 128 * 10000 + 512: return launch_long<512>(p, stream);
    case 128 * 10000 + 128: return launch_long<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_emit(const PoolArgs &p, int head_dim, hipStream_t stream) {
  if (p.batch <= 0) return hipSuccess;
  if (p.groups != 1 || p.first_entry < 1 || !p.shift_kv || !p.shift_sc || p.ape) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)p.batch), block(128);
  switch (head_dim) {
    case 512: hipLaunchKernelGGL((decode_emit_kernel<512, 4>), grid, block, 0, stream, p); break;
    case 128: hipLaunchKernelGGL((decode_emit_kernel<128, 4>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rows_finish(const PoolArgs &p, int head_dim, hipStream_t stream) {
  if (p.groups <= 0) return hipSuccess;
  const dim3 grid((uint32_t)((p.groups + 3) / 4)), block(256);
  switch (head_dim) {
    case 512: hipLaunchKernelGGL(rows_finish_kernel<512>, grid, block, 0, stream, p); break;
    case 128: hipLaunchKernelGGL(rows_finish_kernel<128>, grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pool_boundary(const PoolArgs &p, int64_t row_tiles, int64_t seqlen, int head_dim,
                                hipStream_t stream) {
  if (row_tiles <= 1 || p.groups <= 0) return hipSuccess;
  const dim3 grid((uint32_t)((row_tiles - 1 + 3) / 4)), block(256);
  switch (head_dim) {
    case 512: hipLaunchKernelGGL(pool_boundary_kernel<512>, grid, block, 0, stream, p, row_tiles, seqlen); break;
    case 128: hipLaunchKernelGGL(pool_boundary_kernel<128>, grid, block, 0, stream, p, row_tiles, seqlen); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_state_store(const StateStoreArgs &s, hipStream_t stream) {
  const int64_t total = s.batch * s.state_rows * (s.proj / 4);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(state_store_kernel, dim3((uint32_t)((total + 255) / 256)), dim3(256), 0, stream, s);
  return hipGetLastError();
}

hipError_t launch_decode_finish(const IngestArgs &g, const PoolArgs *pool, int head_dim, hipStream_t stream) {
  if (g.batch <= 0) return hipSuccess;
  const dim3 grid((uint32_t)g.batch), block(256);
  if (!pool) {
    hipLaunchKernelGGL((decode_finish_kernel<512, 4, true, false>), grid, block, 0, stream, g, PoolArgs{});
    return hipGetLastError();
  }
  switch (g.ratio * 10000 + head_dim) {
    case 2 * 10000 + 512:
      hipLaunchKernelGGL((decode_finish_kernel<512, 2, false, true>), grid, block, 0, stream, g, *pool); break;
    case 2 * 10000 + 128:
      hipLaunchKernelGGL((decode_finish_kernel<128, 2, false, true>), grid, block, 0, stream, g, *pool); break;
    case 4 * 10000 + 512:
      hipLaunchKernelGGL((decode_finish_kernel<512, 4, true, true>), grid, block, 0, stream, g, *pool); break;
    case 4 * 10000 + 128:
      hipLaunchKernelGGL((decode_finish_kernel<128, 4, true, true>), grid, block, 0, stream, g, *pool); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fp4_quant(const uint16_t *in, int64_t rows, int64_t width, uint8_t *codes, uint8_t *scales,
                            uint16_t *out, int e8m0, hipStream_t stream) {
  const int64_t n8 = rows * width / 8;
  if (n8 == 0) return hipSuccess;
  const dim3 grid((uint32_t)((n8 + 256 * kQuantChunks - 1) / (256 * kQuantChunks))), block(256);
  if (e8m0 && out) hipLaunchKernelGGL((fp4_quant_kernel<true, true>), grid, block, 0, stream, in, n8, codes, scales, out);
  else if (e8m0) hipLaunchKernelGGL((fp4_quant_kernel<true, false>), grid, block, 0, stream, in, n8, codes, scales, out);
  else if (out) hipLaunchKernelGGL((fp4_quant_kernel<false, true>), grid, block, 0, stream, in, n8, codes, scales, out);
  else hipLaunchKernelGGL((fp4_quant_kernel<false, false>), grid, block, 0, stream, in, n8, codes, scales, out);
  return hipGetLastError();
}

}  // namespace kvc
