// Internal launchers of libkvc.so's kernels. Host code only; not part of the
// C ABI. Each launcher enqueues on `stream` and returns the hipError_t of the
// launch. Shapes are checked by the C-ABI layer before any launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

// C_h[m][n] = sum_k A[m][k] * B_h[n][k] for the two halves h = 0, 1 of the
// output columns (kv with wkv, score with wgate), f32 in and out, fp32 MFMA.
// The K range is cut into `splits` equal parts; split s writes its partial
// sums at C_h + s * c_split_stride. With a16 set (decode only), A is bf16.
// Optionally the second half gets a positional bias row added to each output
// row (one f32 addition): row r of C_1 adds bias1[((r mod bias_seqlen) mod
// bias_ratio) * ldc + n] (the gate logits' bias of token r mod seqlen;
// bias_ratio a power of two).
struct GemmArgs {
  const float *a;       // [m][k], row stride lda
  const float *b0, *b1; // [n_half][k] each, row stride ldb
  float *c0, *c1;       // [m][n_half] each, row stride ldc
  int64_t lda, ldb, ldc;
  int64_t m, n_half, k;
  int32_t splits;
  int64_t c_split_stride;
  const float *bias1;   // [bias_ratio][ldc] or null (splits must be 1)
  int64_t bias_seqlen;
  int32_t bias_ratio;
  // Pooling epilogue (ratio 4, launch_gemm_pool): the kernel computes the
  // kv and score values of both branches of 64 features per column tile and
  // pools every entry inside its row tile into `pooled`; the first entry of
  // each row tile is left to launch_pool_boundary. Rows written to c0 / c1
  // (with the bias on the score plane): the first block of each row tile
  // (branch A), its last block (branch B), and every row from the last
  // complete block of each batch row on (the state's source).
  float *pooled;        // [pool_batch][pool_groups][pool_hd] f32
  int64_t pool_batch, pool_seqlen, pool_groups;
  int32_t pool_hd;
  // bf16 hidden states (launch_gemm_x3*, and decode when set): [m][k], row stride lda
  const uint16_t *a16;
  // three-part weights of launch_gemm_x3* (launch_split_weights' output)
  const uint16_t *bsplit;
  // f16 parts (launch_gemm_h3*): bsplit holds two f16 parts per weight, and
  // the row exponents of the scaled split (x rows: launch_row_exponents,
  // weight rows: launch_split_weights with f16 set)
  const int32_t *xexp, *wexp;
  // f32 matrix cores (launch_gemm, launch_gemm_pool): gemm_rag_floats(m,
  // n_half) f32 where a ragged last row tile keeps its running sum between
  // k segments (tiles with every row inside m keep it in C)
  float *rag;
};

// Prefill tiles need n_half % 128 == 0, k % 32 == 0 and splits == 1 (each
// output summed over the kKSegments k segments defined below); the
// decode shape (bf16 a16 only, the split-K partials of `splits` parts) needs
// n_half % 32 == 0 and k % 16 == 0, no bias.
enum class GemmShape { kPrefill, kDecode };
hipError_t launch_gemm(const GemmArgs &g, GemmShape shape, hipStream_t stream);

// Floats of GemmArgs.rag: 256 rows of every column of both halves.
inline int64_t gemm_rag_floats(int64_t n_half) { return 256 * 2 * n_half; }

// The ratio-4 projection with pooling in the epilogue (fields above):
// b0 = wkv, b1 = wgate ([2 * pool_hd][k] each), m = pool_batch * pool_seqlen,
// needs pool_batch == 1 or pool_seqlen % 4 == 0, k % 32 == 0.
hipError_t launch_gemm_pool(const GemmArgs &g, hipStream_t stream);
// Number of 256-row tiles of launch_gemm_pool (the boundary entries' count + 1).
inline int64_t gemm_pool_row_tiles(int64_t m) { return (m + 255) / 256; }

// bf16 x times f32 weights as three exact bf16 parts (gemm_bf16.hip):
// launch_split_weights writes out[2 n_half][3][k] (bf16 hi, mid, lo of each
// weight) from w0 (rows 0 .. n_half - 1) and w1 (the rest); with pool_hd set
// (ratio 4, n_half = 2 pool_hd) the rows are in the order of the pooling
// kernel's column tiles (see split_weights_kernel). Needs k % 8 == 0,
// 16-byte aligned rows.
struct SplitArgs {
  const float *w0, *w1;  // [n_half][k] each, row stride ldw
  int64_t ldw, n_half, k;
  int32_t pool_hd;       // 0: plain order
  int32_t pool_tile;     // pooling order: split rows per column tile (256 or 128)
  int32_t pool_wn;       // pooling order: columns per wavefront (64 or 128)
  uint16_t *out;
  // f16 set: out[2 n_half][2][k] holds the f16 parts (h, l) of each weight
  // row scaled by 2^exp_out[row] (launch_gemm_h3*), one workgroup per row
  int32_t f16;
  int32_t *exp_out;
};
hipError_t launch_split_weights(const SplitArgs &a, hipStream_t stream);
// Scale exponent e of each of the m rows of x ([m][k], row stride lda, k % 4
// == 0): 2^e brings the row's largest magnitude into [2^14, 2^15); 0 for a
// row of zeros or one holding an infinity (NaN elements are passed over).
hipError_t launch_row_exponents(const float *x, int64_t m, int64_t k, int64_t lda, int32_t *out,
                                hipStream_t stream);
// The prefill projection from a16 and bsplit (plain order), the bias as in
// launch_gemm; n_half % 128 == 0, k % 32 == 0.
hipError_t launch_gemm_x3(const GemmArgs &g, hipStream_t stream);
// As launch_gemm_pool, from a16 and bsplit (pooling order, 256-row tiles).
hipError_t launch_gemm_x3_pool(const GemmArgs &g, hipStream_t stream);
// f32 x (a) times the three-part weights (bsplit) on the bf16 matrix cores:
// x split into three bf16 parts in registers, the six part products of
// magnitude order >= 2^-16 summed in f32. n_half % 128 == 0, k % 32 == 0;
// the pooling variant takes bsplit in pooling order with 128-row tiles.
hipError_t launch_gemm_x6(const GemmArgs &g, hipStream_t stream);
hipError_t launch_gemm_x6_pool(const GemmArgs &g, hipStream_t stream);
// f32 x (a) times the two-part f16 weights (bsplit, wexp) on the f16 matrix
// cores: x rows scaled by 2^xexp and split into two f16 parts in registers,
// the three part products xh wh, xh wl, xl wh summed in f32, the sum scaled
// back by 2^-(xexp + wexp). Shapes and orders as launch_gemm_x6*.
hipError_t launch_gemm_h3(const GemmArgs &g, hipStream_t stream);
hipError_t launch_gemm_h3_pool(const GemmArgs &g, hipStream_t stream);

// Ratio-1 projection: C[m][n] = sum_k A[m][k] * B[n][k], bf16 A and B, f32
// accumulation and output, bf16 MFMA. Needs k % 64 == 0 and n % 128 == 0.
struct GemmBf16Args {
  const uint16_t *a;  // [m][k] bf16, row stride lda
  const uint16_t *b;  // [n][k] bf16, row stride ldb
  float *c;           // [m][n] f32, row stride ldc
  int64_t lda, ldb, ldc;
  int64_t m, n, k;
};
hipError_t launch_gemm_bf16(const GemmBf16Args &g, hipStream_t stream);

// Pools `groups` entries of each batch row from kv/score planes holding a
// sequence of token rows (see the pool kernels for the candidate layout).
struct PoolArgs {
  const float *kv, *sc;       // planes: row t of batch b at b * batch_stride + t * row_stride
  int64_t row_stride, batch_stride;
  int64_t batch, groups;
  int64_t first_entry;        // entry index of output 0 inside the sequence
  int32_t entries_per_wave;
  const float *ape;           // [ratio][row_stride] bias added to score rows, or null
  const float *norm_w;        // [head_dim] or null
  float eps;
  uint16_t *latent;
  float *pooled;
  uint8_t *codes, *scales;
  uint16_t *deq;
  int32_t e8m0;               // codes/scales in the power-of-two, block-32 form
  const float *rope_cs;       // [rows][rope_dim / 2][2] (cos, sin), or null: no RoPE
  int32_t rope_dim;           // rotary slice: the last rope_dim features
  int64_t rope_row0;          // table row of output entry 0 (entry e uses row rope_row0 + e)
  uint16_t *rotated;          // the latent after RoPE, or null
  int64_t out_batch_stride;   // entries per batch row in the outputs
  float *shift_kv, *shift_sc; // ratio 4: move the last block's rows to the previous rows, or null
};
hipError_t launch_pool(const PoolArgs &p, int ratio, int head_dim, hipStream_t stream);

// Decode at ratio 4 when a group completes: the entry of every batch row
// from the state window and the move of the block into the previous-block
// rows, one two-wavefront workgroup per batch row (the move overlapping the
// pooling). p as for launch_pool over the state (groups 1, first_entry 1,
// shift_kv / shift_sc the state planes, no bias).
hipError_t launch_decode_emit(const PoolArgs &p, int head_dim, hipStream_t stream);

// Ratio 1: the per-entry epilogue (bf16 round, RMSNorm, outputs, fp4) of
// `groups` rows of f32 projections, row e at kv + e * row_stride; one entry
// per row (batch 1 in the PoolArgs; sc, ape and the shift are unused).
hipError_t launch_rows_finish(const PoolArgs &p, int head_dim, hipStream_t stream);

// Ratio 4 after launch_gemm_pool: pools the first entry of every row tile but
// the first (entry 64 t of the flattened sequence, when it is not the first
// entry of its batch row) from the plane rows that kernel wrote, into
// p.pooled (only output set). p describes the planes as for launch_pool.
hipError_t launch_pool_boundary(const PoolArgs &p, int64_t row_tiles, int64_t seqlen, int head_dim,
                                hipStream_t stream);

// Writes the carry of a prefill into the state planes (ratio 4: last complete
// block or padding, then the trailing tokens; other ratios: trailing tokens).
struct StateStoreArgs {
  const float *kv, *sc;  // projection planes [batch][seqlen][proj]
  const float *ape;      // [ratio][proj] or null
  float *kv_state, *sc_state;
  int64_t batch, seqlen, proj, state_rows;
  int32_t ratio, overlap;
};
hipError_t launch_state_store(const StateStoreArgs &s, hipStream_t stream);

// Decode: sums the split partial projections of one token per batch row in a
// fixed order, adds the bias row of the slot and writes the state row;
// optionally resets the previous-block rows (ratio 4 at position 0). With
// `pool` (ratios 2 and 4 only), the same launch then pools the state window of
// each batch row (PoolArgs over the state planes, entry 0 of each row).
struct IngestArgs {
  const float *part;      // [splits][2][batch][proj]
  int32_t splits;
  const float *ape;       // [ratio][proj] or null
  float *kv_state, *sc_state;
  int64_t batch, proj, state_rows;
  int32_t slot, state_row, ratio, reset_prev;
};
hipError_t launch_decode_finish(const IngestArgs &g, const PoolArgs *pool, int head_dim, hipStream_t stream);

// The f32 matrix-core projections sum every output over kKSegments k
// segments, the first kKSegments - 1 of 32 * floor(k / (32 kKSegments)) k
// and the last one to k, each one chain of MFMAs from zero, then the chains'
// results in segment order ((p0 + p1) + ...). Prefill (gemm_f32_kernel.h)
// and decode (decode_f32.hip) share it, so they give the same bits.
constexpr int kKSegments = 2;
inline int64_t kseg_length(int64_t k) { return 32 * (k / (32 * kKSegments)); }

// Decode step from f32 x (decode_f32.hip): the projections of one token per
// batch row, summed as the prefill sums them (kKSegments k segments of seg =
// kseg_length(k); one chain when seg is 0),
// and their ingest into the state: the slot's bias row added to the score
// columns, the state row written, and rows [0, reset_rows) reset to (0,
// -inf). The segments run in different workgroups; the last to finish a
// tile (arrival counter in `counters`, zero at rest and left zero) combines
// them.
struct DecodeArgs {
  const float *x;             // [m][k] f32
  const float *w0, *w1;       // wkv, wgate [n_half][k]
  int64_t m, k, n_half;       // batch, dim, proj
  int64_t seg;                // kseg_length(k)
  float *part;                // [kKSegments][m][2 n_half] partial sums of the segments
  uint32_t *counters;         // [decode_f32_tiles(m, n_half)]
  const float *ape;           // [ratio][n_half] or null
  float *kv_state, *sc_state; // [m][state_rows][n_half] each
  int64_t state_rows;
  int32_t slot, state_row, reset_rows;
};
hipError_t launch_decode_f32(const DecodeArgs &d, hipStream_t stream);
// tiles (= arrival counters) of a decode step over m rows, 2 n_half columns
int64_t decode_f32_tiles(int64_t m, int64_t n_half);

// Standalone RoPE of bf16 rows: row r turns its last rope_dim features by
// table row first_row + r. in may equal out.
struct RopeArgs {
  const uint16_t *in;
  uint16_t *out;
  int64_t rows, width;
  int32_t rope_dim;
  const float *rope_cs;  // [.][rope_dim / 2][2]
  int64_t first_row;
};
hipError_t launch_rope(const RopeArgs &a, hipStream_t stream);

// Standalone fp4 round trip of bf16 rows: e4m3 scales per block of 16, or
// (e8m0 set) power-of-two scales per block of 32.
hipError_t launch_fp4_quant(const uint16_t *in, int64_t rows, int64_t width, uint8_t *codes,
                            uint8_t *scales, uint16_t *out, int e8m0, hipStream_t stream);

}  // namespace kvc
