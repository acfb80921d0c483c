/*
 * kvc.h - C ABI of libkvc.so, the MI355X (gfx950) compressor of the
 * DeepSeek-V4.1 compressed-attention KV cache.
 *
 * The compressor turns hidden states x [batch, seqlen, dim] into compressed
 * KV entries, one per `ratio` tokens:
 *   1. kv = x . wkv^T and score = x . wgate^T, f32 weights [proj, dim]
 *      ("Module compress", Functions, linear_f32; "DeepSeek V4.1 . Pool token
 *      pairs", Compressor listing, forward).
 *   2. score += ape[t mod ratio], a positional bias on the gate logits
 *      ("Compressed Sparse Attention . ratio m = 4", Per-channel gated
 *      pooling).
 *   3. Groups of `ratio` tokens. At ratio 4 the groups overlap: each token's
 *      projections hold two branches of head_dim (A = columns [0, hd),
 *      B = [hd, 2 hd)), and entry j pools 8 candidates, the previous block's
 *      branch B then the current block's branch A; entry 0's previous branch is
 *      padding (kv 0, score -inf) ("Compressed Sparse Attention . ratio m = 4",
 *      Why one output uses eight candidates; Tensor-shape walkthrough).
 *   4. Per-feature softmax over the candidates' logits, weighted sum of their
 *      kv values, all in f32 ("DeepSeek V4.1 . Pool token pairs", pooling
 *      formula).
 *   5. Rounding to bf16 and RMSNorm, output rounded to bf16 ("Module
 *      compress", Precision paragraph; Compressor listing, forward).
 *   6. Optionally the cache form of the latent: e2m1 codes with e4m3 scales
 *      per block of 16, and its bf16 dequantisation ("Module compress",
 *      Functions, fp4_quant_e4m3_inplace and to_e2m1_rne).
 * The trailing seqlen mod ratio tokens wait in a caller-owned state, and a
 * decode step emits one entry per completed group (Compressor listing,
 * forward, decode branch; "Compressed Sparse Attention . ratio m = 4", Prefill
 * and decode use the same rule).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers unless marked "host". Arrays are
 *     dense and row-major in the index order given. The caller allocates and
 *     owns all memory; the library allocates no device memory and keeps no
 *     state between calls. Calls on different streams that do not share
 *     buffers may run concurrently.
 *   - bf16 values are passed as their uint16_t bit patterns, e4m3fn scales
 *     and e2m1 codes as bytes.
 *   - Arguments are checked on the host before anything is enqueued; on an
 *     error nothing is enqueued and a negative KVC_E* code is returned.
 *     On success the work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream) and KVC_OK is returned; results are ready when the stream
 *     is synchronised. Device faults surface at that synchronisation.
 *   - "No output yet" (a prefill shorter than ratio, a decode step that does
 *     not complete a group) is not an error: *n_groups / *emitted report it.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *kvc_stream; /* a hipStream_t */

#define KVC_OK 0
#define KVC_EINVAL (-1)       /* a required pointer is NULL, or a size is out of range */
#define KVC_EUNSUPPORTED (-2) /* a valid configuration this library does not implement */
#define KVC_ESPACE (-3)       /* a caller-provided buffer is too small */
#define KVC_EHIP (-4)         /* the HIP runtime rejected a launch */

/* element type of the hidden states x (kvc_config.x_format) */
#define KVC_X_F32 0  /* f32 rows */
#define KVC_X_BF16 1 /* bf16 rows: the model's hidden state */

/* matrix cores of the prefill projection (kvc_config.projection) */
#define KVC_PROJ_AUTO 0       /* default: KVC_PROJ_F32_MFMA for f32 x, KVC_PROJ_BF16_SPLIT for bf16 x */
#define KVC_PROJ_F32_MFMA 1   /* f32 matrix cores (x_format KVC_X_F32 only) */
#define KVC_PROJ_F16_SPLIT 2  /* opt-in emulation: f16 matrix cores on scaled two-part f16 splits (f32 x only) */
#define KVC_PROJ_BF16_SPLIT 3 /* opt-in emulation for f32 x: bf16 matrix cores on three-part bf16 splits */

/* fp4 forms of a compressed entry (kvc_config.fp4_format) */
#define KVC_FP4_E4M3_B16 0 /* the KV latent's form: e4m3fn scale per block of 16 */
#define KVC_FP4_E8M0_B32 1 /* the indexer's form: power-of-two (e8m0) scale per block of 32 */

/* Compressor configuration.
 *   ratio      : 2, 4 or 128 (4 is the overlapped two-branch variant); 1 for
 *                compressor_ratio1_forward only.
 *   head_dim   : latent width hd, 128 or 512.
 *   dim        : hidden width of x, a positive multiple of 32 and at most
 *                2^20 (KVC_EUNSUPPORTED otherwise; ignored when x is NULL).
 *   eps        : RMSNorm epsilon (finite, >= 0).
 *   fp4_format : form of kvc_outputs.codes / scales: KVC_FP4_E4M3_B16 (the
 *                KV latent's, "Module compress", Functions,
 *                fp4_quant_e4m3_inplace) or KVC_FP4_E8M0_B32 (the indexer's,
 *                fp4_quant_e8m0_inplace; Precision paragraph: block 32).
 *   rope_dim   : width of the rotary slice ("Compressed Sparse Attention .
 *                ratio m = 4", Normalize + RoPE + cache; Released Flash
 *                configuration, RoPE sub-dimension 64), or 0 for no RoPE.
 *                Even, at most head_dim; not offered at ratio 1. With RoPE,
 *                the entry's last rope_dim features turn as pairs (2i, 2i+1)
 *                by row j of kvc_weights.rope_cs for compressed entry j:
 *                (a, b) -> (a c - b s, a s + b c), each exact value rounded
 *                once to bf16; the rotated entry goes to kvc_outputs.rotated
 *                and is what the fp4 outputs encode, while latent stays the
 *                unrotated compressor output.
 *   x_format   : KVC_X_F32 or KVC_X_BF16, the element type of x in
 *                compressor_prefill and compressor_decode_step (ratio > 1).
 *                The compressor promotes the model's bf16 hidden state to f32
 *                before its f32 projections ("DeepSeek V4.1 . Pool token
 *                pairs", Compressor listing, forward); with KVC_X_BF16 the
 *                caller passes that bf16 state. Ignored by
 *                compressor_ratio1_forward, whose x is always bf16.
 *   projection : how compressor_prefill computes the f32 products x . w^T:
 *                KVC_PROJ_F32_MFMA (what KVC_PROJ_AUTO, 0, selects for f32
 *                x): on the f32 matrix cores. Each output is the sum of two
 *                halves of the hidden width, p0 over k in [0, ks) and p1 over
 *                [ks, dim) with ks = 32 * floor(dim / 64), each accumulated
 *                from zero in one fixed k order, then p0 + p1 in one f32
 *                addition (p1 alone when ks is 0). A decode step with f32 x
 *                computes its projections as the same two sums, so decode
 *                and prefill give the same bits for the same tokens.
 *                The other two are opt-in emulations of the f32 products on
 *                16-bit matrix cores, with f32 accumulation:
 *                KVC_PROJ_F16_SPLIT (f32 x only): every row of x and every
 *                weight row is scaled by the power of two that brings its
 *                largest magnitude into [2^14, 2^15); each scaled value y
 *                splits into h = f16(y) and l = f16(y - h) (y - h - l at most
 *                2^-22 |y|, or 2^-40 of the row's largest magnitude where l
 *                falls below the f16 normal range); the three part products
 *                xh wh + xh wl + xl wh are summed (xl wl, left out, is at most
 *                2^-22 |x w|) and the sum is scaled back exactly.
 *                KVC_PROJ_BF16_SPLIT: on the bf16 matrix cores from the exact
 *                split of each f32 weight into three bf16 parts (hi, mid, lo:
 *                bits cleared, so w = hi + mid + lo); bf16 x then gives exact
 *                products (x . hi + x . mid + x . lo), and f32 x is split the
 *                same way and the six part products of size >= 2^-16 |x w|
 *                are summed (the three left out total below 2^-21 |x w|).
 *                KVC_PROJ_AUTO selects it for bf16 x (whose products with
 *                the three parts are exact).
 *                KVC_PROJ_F16_SPLIT and KVC_PROJ_F32_MFMA need x_format
 *                KVC_X_F32 (KVC_EINVAL otherwise). Every error above lies far
 *                inside the f32 summation's own bound (K 2^-24 sum |x w|).
 *                Decode steps always use the f32 matrix cores.
 * proj = 2 * head_dim at ratio 4, head_dim otherwise: the width of each
 * projection plane. */
typedef struct kvc_config {
    int32_t ratio;
    int32_t head_dim;
    int64_t dim;
    float eps;
    int32_t fp4_format;
    int32_t rope_dim;
    int32_t x_format;
    int32_t projection;
} kvc_config;

/* Weights (device, f32).
 *   wkv, wgate : [proj][dim]; required whenever x is not NULL.
 *   ape        : [ratio][proj] positional bias of the gate logits, or NULL
 *                (no bias).
 *   norm_w     : [head_dim] RMSNorm weight, or NULL (all ones).
 *   rope_cs    : [rope_rows][rope_dim / 2][2] (cos, sin) of each compressed
 *                entry's rotation ("Module compress", Functions,
 *                yarn_freqs_cis: the caller builds it from its own theta and
 *                YaRN parameters, row j for compressed entry j); required when
 *                rope_dim > 0 and an entry is written, else ignored.
 *   rope_rows  : rows of rope_cs; every entry written needs j < rope_rows. */
typedef struct kvc_weights {
    const float *wkv;
    const float *wgate;
    const float *ape;
    const float *norm_w;
    const float *rope_cs;
    int64_t rope_rows;
} kvc_weights;

/* Outputs (device). Each is written iff its pointer is not NULL; G is the
 * number of entries of the call (groups for a prefill, 1 for an emitting
 * decode step).
 *   latent  : [batch][G][head_dim] bf16, the RMSNorm output.
 *   pooled  : [batch][G][head_dim] f32, the pooled value before rounding.
 *   codes   : [batch][G][head_dim / 2] e2m1 codes of the latent, two per
 *             byte, element 2k in the low nibble, sign in bit 3 of a nibble.
 *   scales  : [batch][G][head_dim / 16] e4m3fn scale of each block of 16, or
 *             with KVC_FP4_E8M0_B32 [batch][G][head_dim / 32] e8m0 scale
 *             bytes (2^(byte - 127)) of each block of 32.
 *   dequant : [batch][G][head_dim] bf16, codes times scales.
 *   rotated : [batch][G][head_dim] bf16, the latent after RoPE (requires
 *             rope_dim > 0). With RoPE, codes / scales / dequant encode this
 *             rotated entry. */
typedef struct kvc_outputs {
    uint16_t *latent;
    float *pooled;
    uint8_t *codes;
    uint8_t *scales;
    uint16_t *dequant;
    uint16_t *rotated;
} kvc_outputs;

/* proj for `cfg`, or a negative KVC_E* code if cfg is invalid. */
int64_t kvc_proj_width(const kvc_config *cfg);

/* Rows of each state plane: 2 * ratio at ratio 4, ratio otherwise; or a
 * negative KVC_E* code. */
int64_t kvc_state_rows(const kvc_config *cfg);

/* f32 elements of the workspace compressor_prefill needs: the projection
 * planes, 2 * batch * seqlen * proj; at ratio 4 the f32 pooled entries,
 * batch * (seqlen / 4) * head_dim (used when the projection and the pooling
 * run as one kernel: a smaller workspace runs them separately); then, by
 * projection: on the f32 matrix cores (KVC_PROJ_F32_MFMA, the default for
 * f32 x) the running sums of a ragged last row tile, 256 * 2 * proj; for the
 * opt-in KVC_PROJ_F16_SPLIT two f16 weight parts and the scale exponents of
 * the weight rows and of x's rows, 2 * proj * dim + 2 * proj + batch * seqlen
 * rounded up to a multiple of 4; for KVC_PROJ_BF16_SPLIT (and KVC_PROJ_AUTO
 * with bf16 x) three bf16 weight parts, 3 * proj * dim. Or a negative KVC_E*
 * code. */
int64_t kvc_prefill_workspace_floats(const kvc_config *cfg, int64_t batch, int64_t seqlen);

/* f32 elements of the workspace compressor_decode_step needs, or a negative
 * code. It holds the partial sums of the projection and, after them, the
 * arrival counters of its two k halves (one per tile of 32 batch rows x 32
 * columns). The workspace must be zero-filled before the first call that
 * uses it; every completed call leaves the counters zero again, so the same
 * workspace serves any number of steps, graph replays included. Where a
 * call finds a counter that is not zero (a workspace that was not
 * zero-filled), the state row it writes is NaN in that tile rather than
 * silently wrong; zero-fill the workspace again before going on. The same
 * size for either x_format. */
int64_t kvc_decode_workspace_floats(const kvc_config *cfg, int64_t batch);

/* Compressor forward at start_pos == 0 (prefill) over `seqlen` tokens of
 * `batch` rows ("DeepSeek V4.1 . Pool token pairs", Compressor listing,
 * forward, prefill branch; the overlap of "Compressed Sparse Attention .
 * ratio m = 4").
 *   x            : [batch][seqlen][dim] f32, or bf16 with KVC_X_BF16 (16-byte
 *                  aligned either way), or NULL. NULL means the caller
 *                  has put the projections (without bias) in `workspace`:
 *                  the kv plane [batch][seqlen][proj] followed by the score
 *                  plane [batch][seqlen][proj]; no weights are read then
 *                  except ape and norm_w.
 *   batch        : >= 1.   seqlen : >= 0.
 *   workspace    : f32, at least 2 * batch * seqlen * proj elements, and
 *                  with x all kvc_prefill_workspace_floats() elements
 *                  (KVC_ESPACE otherwise); receives the two projection planes
 *                  when x is not NULL (the score plane then with the
 *                  positional bias added; at ratio 4 with the fused kernel,
 *                  only the rows the state and the row tiles' first entries
 *                  read hold projections, and the other rows intermediate
 *                  values such as the first k half's partial sums).
 *   kv_state,
 *   score_state  : [state_batch][kvc_state_rows()][proj] f32 each, or both
 *                  NULL (nothing carried). Rows of batch row b are written as
 *                  the decode continuation needs them: non-overlapped, rows
 *                  [0, seqlen mod ratio) get the trailing tokens; at ratio 4,
 *                  rows [0, 4) get the last complete block (kv 0 / score -inf
 *                  when there is none) and rows [4, 4 + seqlen mod 4) the
 *                  trailing tokens. Scores are stored with the bias added.
 *   state_batch  : capacity of the state planes in batch rows (>= batch).
 *   out          : outputs with G = seqlen / ratio (host struct; may be NULL
 *                  to compute only projections and state).
 *   n_groups     : host, optional; receives seqlen / ratio (0: no entry).
 * Errors: KVC_EINVAL, KVC_EUNSUPPORTED, KVC_ESPACE, KVC_EHIP. */
int compressor_prefill(const kvc_config *cfg, const kvc_weights *w, const void *x, int64_t batch,
                       int64_t seqlen, float *workspace, int64_t workspace_floats,
                       float *kv_state, float *score_state, int64_t state_batch, const kvc_outputs *out,
                       int64_t *n_groups, kvc_stream stream);

/* One decode step: one token per batch row at position start_pos
 * (Compressor listing, forward, decode branch). The token fills slot
 * start_pos mod ratio of the state; when (start_pos + 1) mod ratio == 0 the
 * group is pooled and one entry per batch row is written to `out` (G = 1);
 * at ratio 4 the current block then becomes the previous one. start_pos == 0
 * is a prefill of one token, which resets the carried block.
 * Launches: from f32 x, one kernel computes the projections (summed exactly
 * as compressor_prefill's f32 matrix cores sum them, so the entries equal a
 * prefill's bit for bit) and writes the state row; a step that completes a
 * group launches the pooling kernel after it (at ratio 4 the same kernel
 * moves the block, while it pools). From bf16 x or given
 * projections: the projection (bf16 x), then one kernel that ingests and,
 * at ratios 2 and 4, pools.
 *   x            : [batch][dim] f32, or bf16 with KVC_X_BF16 (one token per
 *                  row), or NULL: then the
 *                  caller has put the token's projections (without bias) in
 *                  workspace[0 : 2 * batch * proj] as the kv rows
 *                  [batch][proj] followed by the score rows [batch][proj].
 *   start_pos    : >= 0, the token's position in its sequence.
 *   workspace    : f32, >= kvc_decode_workspace_floats() elements, its
 *                  counters zero (see there). Two calls that share a
 *                  workspace must not run concurrently.
 *   kv_state,
 *   score_state  : required, as for compressor_prefill, holding the carry
 *                  of the previous calls of this sequence.
 *   emitted      : host, optional; receives 1 if entries were written, else 0.
 * Errors: as compressor_prefill. */
int compressor_decode_step(const kvc_config *cfg, const kvc_weights *w, const void *x, int64_t batch,
                           int64_t start_pos, float *workspace, int64_t workspace_floats,
                           float *kv_state, float *score_state, int64_t state_batch,
                           const kvc_outputs *out, int32_t *emitted, kvc_stream stream);

/* compressor_decode_step for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same step, with the same kernels and results, but no
 * workspace argument. Its partial sums and arrival counters live in a
 * scratch array inside the library, 4 MiB + 16 KiB of device memory that
 * each GPU the library runs on holds until the process ends (the counters
 * start at zero and every completed step leaves them zero). Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (different
 * streams, or different threads without ordering) race and give undefined
 * results; serialise them.
 *   Arguments as compressor_decode_step, except that x is required (given
 *   projections need the caller's workspace: KVC_EINVAL).
 *   Limits: the step's partial sums (kvc_decode_workspace_floats() less
 *   its counters) must fit in 2^20 floats and its counters in 4096: batch
 *   <= 256 at proj 1024, 512 at proj 512, 1024 at proj 256; KVC_ESPACE
 *   beyond. KVC_EHIP if the scratch address cannot be resolved.
 * Nothing is allocated by the call (no hipMalloc or allocating library
 * routine). */
int compressor_decode_step_noalloc(const kvc_config *cfg, const kvc_weights *w, const void *x, int64_t batch,
                                   int64_t start_pos, float *kv_state, float *score_state, int64_t state_batch,
                                   const kvc_outputs *out, int32_t *emitted, kvc_stream stream);

/* f32 elements of the workspace compressor_ratio1_forward needs:
 * tokens * head_dim; or a negative KVC_E* code (cfg->ratio must be 1). */
int64_t kvc_ratio1_workspace_floats(const kvc_config *cfg, int64_t tokens);

/* The ratio-1 compressor ("DeepSeek V4.1 . Pool token pairs", Compressor
 * listing, __init__ and the ratio-1 branch of forward; "Module compress",
 * CompressorWeights): no gate, no pooling and no state, every token is one
 * entry: latent = RMSNorm(bf16(x . wkv^T)) with bf16 x and bf16 wkv, the
 * products summed in f32. Prefill and decode are the same call.
 *   cfg          : ratio 1 (any other ratio: KVC_EINVAL); head_dim 128 or
 *                  512; dim a positive multiple of 64, at most 2^20.
 *   wkv          : [head_dim][dim] bf16.
 *   norm_w       : [head_dim] f32 RMSNorm weight, or NULL (all ones).
 *   x            : [tokens][dim] bf16 (batch rows and positions flattened).
 *   tokens       : >= 0 (0: nothing is enqueued).
 *   workspace    : f32, >= kvc_ratio1_workspace_floats() elements; receives
 *                  the f32 projections [tokens][head_dim].
 *   out          : outputs with batch 1 and G = tokens; `pooled` receives the
 *                  f32 projection (before the bf16 rounding). May be NULL to
 *                  compute only the projections.
 * Errors: KVC_EINVAL, KVC_EUNSUPPORTED, KVC_ESPACE, KVC_EHIP. */
int compressor_ratio1_forward(const kvc_config *cfg, const uint16_t *wkv, const float *norm_w,
                              const uint16_t *x, int64_t tokens, float *workspace,
                              int64_t workspace_floats, const kvc_outputs *out, kvc_stream stream);

/* The latent's fp4 round trip ("Module compress", Functions,
 * fp4_quant_e4m3_inplace; to_e2m1_rne; Constants, LATENT_BLOCK) on
 * [rows][width] bf16 values. Each run of 16 consecutive values of a row
 * shares one scale: the largest magnitude M of the run, raised to 6 * 2^-9
 * when smaller, is divided by 6 (IEEE f32 division) and rounded to the
 * nearest e4m3fn value (ties to even). Each value divided by that scale maps
 * to the nearest e2m1 code (ties to the even code, saturating at 6, the sign
 * bit kept even for a zero code); the dequantised value is the code's value
 * times the scale, which bf16 holds exactly.
 *   in     : [rows][width] bf16.   rows >= 0, width > 0 and width % 16 == 0.
 *   codes  : [rows][width / 2] bytes (layout as kvc_outputs.codes), or NULL.
 *   scales : [rows][width / 16] e4m3fn bytes, or NULL.
 *   out    : [rows][width] bf16 dequantised values, or NULL; may equal `in`
 *            (in place). Other overlaps are not allowed.
 * Errors: KVC_EINVAL, KVC_EHIP. */
int latent_fp4_quant(const uint16_t *in, int64_t rows, int64_t width, uint8_t *codes,
                     uint8_t *scales, uint16_t *out, kvc_stream stream);

/* The indexer's fp4 round trip ("Module compress", Functions,
 * fp4_quant_e8m0_inplace; Constants, FP4_BLOCK; Precision paragraph: the
 * indexer's q and k use power-of-two scales in blocks of 32) on [rows][width]
 * bf16 values. Each run of 32 consecutive values of a row shares one scale
 * 2^e: e is the least integer with 2^e >= M / 6 (IEEE f32 division), M the
 * run's largest magnitude raised to 6 * 2^-126 when smaller (so M / 6 is a
 * normal f32). Codes, their sign and the dequantised values follow the rule
 * of latent_fp4_quant with this scale.
 *   in     : [rows][width] bf16.   rows >= 0, width > 0 and width % 32 == 0.
 *   codes  : [rows][width / 2] bytes (layout as kvc_outputs.codes), or NULL.
 *   scales : [rows][width / 32] e8m0 bytes (e + 127), or NULL.
 *   out    : [rows][width] bf16 dequantised values, or NULL; may equal `in`.
 * Errors: KVC_EINVAL, KVC_EHIP. */
int indexer_fp4_quant(const uint16_t *in, int64_t rows, int64_t width, uint8_t *codes,
                      uint8_t *scales, uint16_t *out, kvc_stream stream);

/* RoPE of [rows][width] bf16 latent rows, the step between the norm and the
 * cache ("Compressed Sparse Attention . ratio m = 4", Normalize + RoPE +
 * cache): row r's last rope_dim features turn as pairs (2i, 2i+1) by
 * rope_cs row first_row + r, (a, b) -> (a c - b s, a s + b c), each exact
 * value rounded once to bf16 (round to nearest even); the same rotation the
 * compressor entry points apply with kvc_config.rope_dim.
 *   in, out   : [rows][width] bf16; out may equal in (in place), other
 *               overlaps are not allowed.
 *   rows >= 0; width > 0 and even; rope_dim even, 0 < rope_dim <= width.
 *   rope_cs   : [rope_rows][rope_dim / 2][2] f32 (cos, sin);
 *               first_row + rows <= rope_rows.
 * Errors: KVC_EINVAL, KVC_EHIP. */
int latent_rope(const uint16_t *in, int64_t rows, int64_t width, int32_t rope_dim, const float *rope_cs,
                int64_t rope_rows, int64_t first_row, uint16_t *out, kvc_stream stream);

/* Measurement hook (for benchmarks and profilers; no effect on results).
 * start and stop are hipEvent_t handles the caller created. The next
 * compressor_prefill or compressor_decode_step call made by the calling
 * thread records start on its stream immediately before it launches its
 * projection kernel (the GEMM, which at ratio 4 may also pool and, in a
 * decode step from f32 x, also writes the state row) and stop immediately
 * after, then forgets both; a call that launches no projection forgets them
 * too. Both NULL clears a pending request. Errors: KVC_EINVAL (only one of
 * the two NULL); a failed record makes the compressor call return
 * KVC_EHIP. */
int kvc_time_next_projection(void *start, void *stop);

/* A static description of a KVC_* code. */
const char *kvc_strerror(int code);

/* Library version string. */
const char *kvc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
