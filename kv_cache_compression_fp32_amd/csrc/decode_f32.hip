// Decode step from f32 hidden states: the token's projections and their
// ingest into the state, one launch per step (gfx950, wave64).
//
// One token per batch row: kv = x . wkv^T, score = x . wgate^T ("Module
// compress", Functions, linear_f32; "DeepSeek V4.1 . Pool token pairs",
// Compressor listing, forward, decode branch), summed exactly as the prefill
// projection sums them (gemm_f32_kernel.h): the kKSegments k segments of
// kvc_launch.h, each one chain of v_mfma_f32_16x16x4_f32 from zero over
// increasing 16-k chunks, k-slot q of MFMA t holding k = chunk + 4 q + t,
// then (p0 + p1) + .. in segment order. So a decode step and a prefill over
// the same tokens write the same bits ("Compressed Sparse Attention . ratio
// m = 4", Prefill and decode use the same rule).
//
// Work split: a workgroup of TM / 8 wavefronts computes a TM x 32 tile (batch
// rows x output columns) over one k segment, wavefront w owning the 16 x 16
// fragment (w / 2, w % 2). The segments of a tile run in different
// workgroups (64 rows x 2048 columns in two segments make 256 workgroups of
// 32 x 32). Each writes its segment's partial sums to the workspace with
// device-coherent stores; an arrival counter per tile (workspace, zero at
// rest) tells the last one to arrive, which reads the other partials with
// device-coherent loads, adds them in segment order, adds the bias row of
// the token's slot to the score columns, writes the state row and resets
// the counter, so the next step (or a graph replay) finds it zero. No
// workgroup waits for another, and no cache-wide fence is needed: every
// value that crosses workgroups is written and read coherently, and a
// wavefront's stores have completed before its workgroup's arrival.
//
// Operands reach LDS through buffer loads that write it directly (no
// registers): a stage is BK k of the tile's TM x rows and 32 weight rows,
// the 16-byte group q of row r at position q ^ (r & 15) (stages of 64 k;
// q ^ (r & 7) with 32 k), so the fragment reads of 16 neighbouring rows hit
// 16 distinct bank groups. NST stage buffers, the loads NST - 1 stages
// ahead. One wavefront per SIMD runs one dependent chain, so whatever the
// wavefront issues between two chunks of MFMAs delays the chain: the loads
// go out one per chunk, between the MFMAs; the fragment reads of stage s + 1
// go out after the barrier that ends step s and drain while the chain of
// step s + 1 runs, each chunk waiting only for its own two reads. LDS reads
// are inline asm, which the compiler does not track: it would otherwise
// wait for every load in flight into any stage buffer before each of them.
// Each wait is tied to the values it covers.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gemm_common.h"
#include "kvc_launch.h"

namespace kvc {
namespace {

using gemm::buffer_load_lds;
using gemm::f4;
using gemm::i32x4;
using gemm::lds_u32;
using gemm::make_rsrc;
using gemm::uniform_rsrc;
using gemm::xcd_remap;

constexpr int kTN = 32;  // output columns per workgroup

typedef __attribute__((address_space(3))) float lds_f32;

// s_waitcnt immediate waiting until at most n vector memory operations of
// this wavefront are in flight (lgkmcnt and expcnt not waited on)
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

__device__ __forceinline__ void barrier_no_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int TM, int BK, int NST>
__global__ __launch_bounds__(TM / 8 * 64) void decode_f32_kernel(DecodeArgs d) {
  constexpr int kTM = TM, kWaves = TM / 8;  // one 16 x 16 fragment per wavefront
  constexpr int P = BK / 4;              // 16-byte groups per row piece
  constexpr int RPI = 64 / P;            // rows per load instruction
  // row r's 16-byte group q sits at position q ^ (r & SWM): with 16 or more
  // groups per row (stages of 64 k or more) the 16 rows of a fragment read
  // land on 16 distinct 16-byte bank groups (measured on gfx950: 1 us per
  // step faster than spreading 8 rows, whose pairs r, r + 8 then share banks)
  constexpr int SWM = P >= 16 ? 15 : 7;
  constexpr int XI = kTM / RPI;          // load instructions per stage: x
  constexpr int WI = kTN / RPI;          //                              weights
  constexpr int XPW = (XI + kWaves - 1) / kWaves, WPW = (WI + kWaves - 1) / kWaves;  // per wavefront
  constexpr int KK = BK / 16;            // 16-k chunks per stage
  static_assert(XI * RPI == kTM && WI * RPI == kTN && XI % kWaves == 0 && (WI % kWaves == 0 || WI < kWaves),
                "stage / wavefront mismatch");
  static_assert(NST >= 3, "a step loads into the buffer of the stage before it, read one step earlier");
  __shared__ __attribute__((aligned(16))) float xs[NST][kTM * BK];
  __shared__ __attribute__((aligned(16))) float ws[NST][kTN * BK];
  __shared__ uint32_t s_arrival;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // tile order: batch row tile fastest, then k segment, then column tile;
  // each XCD walks a contiguous range, so the segments of a tile meet in
  // one L2 and share the tile's x rows there
  const int64_t m_tiles = (d.m + kTM - 1) / kTM;
  const int segs = d.seg > 0 ? kKSegments : 1;
  const uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
  const int64_t mt = id % m_tiles;
  const int seg = (int)((id / m_tiles) % segs);
  const int64_t nt = id / (m_tiles * segs);
  const int64_t n_glob = nt * kTN;
  const bool second = n_glob >= d.n_half;
  const int64_t n0 = second ? n_glob - d.n_half : n_glob;
  const float *W = second ? d.w1 : d.w0;
  const int64_t m0 = mt * kTM;
  const int64_t kbase = segs == 1 ? 0 : seg * d.seg;
  const int64_t klen = segs == 1 ? d.k : (seg < kKSegments - 1 ? d.seg : d.k - (kKSegments - 1) * d.seg);
  const int stages = (int)(klen / BK);
  const int64_t a_rows = d.m - m0 < kTM ? d.m - m0 : kTM;
  // the bias of this lane's output column for the ingest, loaded ahead of
  // the operands so that it has landed by the end
  const int64_t c = n0 + 16 * (wave & 1) + (lane & 15);
  const bool has_bias = second && d.ape;
  float bias = has_bias ? d.ape[(int64_t)d.slot * d.n_half + c] : 0.0f;

  // buffer resources from the tile's first row at the segment's first k
  const i32x4 a_rsrc = uniform_rsrc(make_rsrc(d.x + m0 * d.k + kbase, (uint32_t)((a_rows * d.k - kbase) * 4)));
  const i32x4 b_rsrc = uniform_rsrc(make_rsrc(W + n0 * d.k + kbase, (uint32_t)((kTN * d.k - kbase) * 4)));
  // x load u of wavefront w fills rows RPI (XPW w + u) + lane / P, weight
  // load u rows RPI (WPW w + u) + lane / P (with fewer weight loads than
  // wavefronts, wavefront w repeats load w mod WI: same bytes to the same
  // place, so every wavefront has the same count in flight); LDS position
  // lane % P holds the row's group (lane % P) ^ (row & SWM); rows past the
  // batch read its last row (computed, never stored)
  const int rsub = lane / P, pos = lane % P;
  uint32_t a_off[XPW], b_off[WPW];
  int a_row0[XPW], b_row0[WPW];
#pragma unroll
  for (int u = 0; u < XPW; ++u) {
    a_row0[u] = RPI * (XPW * wave + u);
    const int r = a_row0[u] + rsub;
    const int64_t rr = r < a_rows ? r : a_rows - 1;
    a_off[u] = (uint32_t)((rr * d.k + 4 * (pos ^ (r & SWM))) * 4);
  }
#pragma unroll
  for (int u = 0; u < WPW; ++u) {
    b_row0[u] = RPI * (WI < kWaves ? wave % WI : WPW * wave + u);
    const int r = b_row0[u] + rsub;
    b_off[u] = (uint32_t)(((int64_t)r * d.k + 4 * (pos ^ (r & SWM))) * 4);
  }
  // load u of stage s into stage buffer buf: the x loads, then the weight loads
  auto issue_one = [&](int s, int buf, int u) {
    const int32_t koff = s * BK * 4;
    if (u < XPW)
      buffer_load_lds(a_rsrc, (lds_u32 *)(&xs[buf][a_row0[u] * BK]), 16, (int32_t)a_off[u], koff, 0, 0);
    else
      buffer_load_lds(b_rsrc, (lds_u32 *)(&ws[buf][b_row0[u - XPW] * BK]), 16, (int32_t)b_off[u - XPW], koff, 0,
                      0);
  };
  constexpr int PER_STAGE = XPW + WPW;  // loads in flight per stage and wavefront

  const int fi = wave >> 1, fj = wave & 1, row_in = lane & 15, slot = lane >> 4;
  const int ra = 16 * fi + row_in, rb = 16 * fj + row_in;
  // chunk kk of a stage: k = 16 kk + 4 slot .. + 3 of rows ra (x) and rb (w)
  auto read = [&](int buf, f4(&af)[KK], f4(&bf)[KK]) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int q = 4 * kk + slot;
      const uint32_t aa = (uint32_t)(uintptr_t)(const lds_f32 *)(&xs[buf][ra * BK + 4 * (q ^ (ra & SWM))]);
      const uint32_t ba = (uint32_t)(uintptr_t)(const lds_f32 *)(&ws[buf][rb * BK + 4 * (q ^ (rb & SWM))]);
      asm volatile("ds_read_b128 %0, %1" : "=v"(af[kk]) : "v"(aa));
      asm volatile("ds_read_b128 %0, %1" : "=v"(bf[kk]) : "v"(ba));
    }
  };
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  // step s: the chain over stage s, whose fragments were read at the end of
  // the previous step. One load of stage s + NST - 1 goes out before each
  // chunk's MFMAs (into the buffer of stage s - 1: every wavefront finished
  // reading it before the previous step's barrier; past the last stage the
  // last one is loaded again into a buffer nobody reads, which keeps the wait
  // counts fixed), and each chunk waits only for its own two fragment reads
  // (a wavefront's LDS reads complete in order), so the reads of a stage
  // drain while the chain runs. Then, once every wavefront's loads of stage
  // s + 1 have landed, its fragments are read.
  auto step = [&](int s, f4(&ca)[KK], f4(&cb)[KK], f4(&na)[KK], f4(&nb)[KK]) {
    const int ahead = s + NST - 1;
    const int sa = ahead < stages ? ahead : stages - 1, ba = ahead % NST;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int u = kk * PER_STAGE / KK; u < (kk + 1) * PER_STAGE / KK; ++u) issue_one(sa, ba, u);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(ca[kk]), "+v"(cb[kk]) : "n"(2 * (KK - 1 - kk)));
#pragma unroll
      for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ca[kk][t], cb[kk][t], acc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((NST - 2) * PER_STAGE));  // this wavefront's stage s + 1 landed
    barrier_no_fence();                                           // every wavefront's
    if (s + 1 < stages) read((s + 1) % NST, na, nb);
    __builtin_amdgcn_sched_barrier(0);
  };

  f4 a0[KK], b0[KK], a1[KK], b1[KK];
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
#pragma unroll
    for (int u = 0; u < PER_STAGE; ++u) issue_one(s < stages ? s : stages - 1, s, u);
  // the bias is needed only at the end; it was loaded before the operands
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((NST - 2) * PER_STAGE));  // stage 0 (and the bias)
  asm volatile("" : "+v"(bias));
  barrier_no_fence();
  read(0, a0, b0);
  for (int s = 0; s < stages; s += 2) {
    step(s, a0, b0, a1, b1);
    if (s + 1 < stages) step(s + 1, a1, b1, a0, b0);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // no load into LDS outlives the workgroup

  // accumulator r of this lane: batch row m0 + 16 fi + 4 slot + r, column
  // n_glob + 16 fj + row_in of the [2 n_half] output row (kv then score)
  const int64_t ncols = 2 * d.n_half;
  const int64_t col = n_glob + 16 * fj + row_in;
  const int64_t row0 = m0 + 16 * fi + 4 * slot;
  float tot[4] = {acc[0], acc[1], acc[2], acc[3]};
  if (segs > 1) {
    const int64_t plane = d.m * ncols;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (row0 + r < d.m)
        __hip_atomic_store(d.part + seg * plane + (row0 + r) * ncols + col, acc[r], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wavefront's partial sums are stored
    __syncthreads();                           // and every wavefront's
    uint32_t *counter = d.counters + nt * m_tiles + mt;
    if (threadIdx.x == 0) s_arrival = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t arrived = s_arrival;
    if (arrived + 1 < (uint32_t)segs) return;  // another segment finishes the tile
    // a counter that was not zero at the call: the caller's workspace was not
    // zero-filled; the state row turns NaN rather than silently wrong
    const bool bad = arrived + 1 != (uint32_t)segs;
    // every segment's partial sums (the own ones too, as stored above), all
    // loads in flight at once; rows past the batch read the last row
    float p[kKSegments][4];
#pragma unroll
    for (int sg = 0; sg < kKSegments; ++sg)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t rr = row0 + r < d.m ? row0 + r : d.m - 1;
        p[sg][r] = __hip_atomic_load(d.part + sg * plane + rr * ncols + col, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float t = p[0][r];
#pragma unroll
      for (int sg = 1; sg < kKSegments; ++sg) t = t + p[sg][r];  // (p0 + p1) + ..
      tot[r] = bad ? __builtin_nanf("") : t;
    }
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the ingest: the bias row of the token's slot joins the gate logits in
  // one f32 addition, then the state row (and at ratio 4 from position 0 the
  // previous block's padding)
  float *state = second ? d.sc_state : d.kv_state;
  const float fill = second ? -INFINITY : 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t row = row0 + r;
    if (row >= d.m) continue;
    const float v = has_bias ? tot[r] + bias : tot[r];
    float *srow = state + row * d.state_rows * d.n_half;
    srow[(int64_t)d.state_row * d.n_half + c] = v;
    for (int i = 0; i < d.reset_rows; ++i) srow[(int64_t)i * d.n_half + c] = fill;
  }
}

template <int TM, int BK, int NST>
hipError_t launch(const DecodeArgs &d, hipStream_t stream) {
  const int64_t tiles = ((d.m + TM - 1) / TM) * (2 * d.n_half / kTN) * (d.seg > 0 ? kKSegments : 1);
  hipLaunchKernelGGL((decode_f32_kernel<TM, BK, NST>), dim3((uint32_t)tiles), dim3(TM / 8 * 64), 0, stream, d);
  return hipGetLastError();
}

constexpr int kDecTM = 32;  // batch rows per workgroup

}  // namespace

int64_t decode_f32_tiles(int64_t m, int64_t n_half) { return ((m + kDecTM - 1) / kDecTM) * (2 * n_half / kTN); }

hipError_t launch_decode_f32(const DecodeArgs &d, hipStream_t stream) {
  if (d.m <= 0) return hipSuccess;
  // whole 32-column tiles, 32-k granules, and tile rows addressable with
  // 32-bit buffer offsets
  if (d.n_half % kTN != 0 || d.k % 32 != 0 || d.seg != kseg_length(d.k) || d.k <= 0 ||
      (int64_t)kDecTM * d.k * 4 > INT32_MAX || (d.seg > 0 && !d.part) || !d.counters || d.slot < 0 ||
      d.state_row < 0 || d.state_row >= d.state_rows || d.reset_rows < 0 || d.reset_rows > d.state_rows)
    return hipErrorInvalidValue;
  // stages of 64 k when every segment is whole stages, else of 32 k (both
  // 64 KiB of LDS, so two workgroups share a CU once the tiles outnumber
  // the CUs)
  const int64_t last = d.k - (kKSegments - 1) * d.seg;
  const bool wide = d.seg > 0 && d.seg % 64 == 0 && last % 64 == 0;
  return wide ? launch<kDecTM, 64, 4>(d, stream) : launch<kDecTM, 32, 8>(d, stream);
}

}  // namespace kvc
