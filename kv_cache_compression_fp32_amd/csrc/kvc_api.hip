// C ABI of libkvc.so (declared in include/kvc.h): argument checks and the
// launch sequence of each entry point. Everything runs in this library's
// kernels on the caller's stream; nothing is allocated and nothing is kept
// between calls.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "kvc.h"
#include "kvc_launch.h"

namespace {

constexpr int64_t kAlign = 16;  // bytes; every device pointer is accessed in 16-byte vectors
// hidden width limit: a 256-row tile of x (or of a weight) must be addressable
// with 32-bit byte offsets by the projection kernel's buffer loads
constexpr int64_t kMaxDim = int64_t(1) << 20;

bool aligned(const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

int check_common(const kvc_config *cfg) {
  if (!cfg) return KVC_EINVAL;
  if (!(cfg->eps >= 0.0f) || !isfinite(cfg->eps)) return KVC_EINVAL;
  if (cfg->fp4_format != KVC_FP4_E4M3_B16 && cfg->fp4_format != KVC_FP4_E8M0_B32) return KVC_EINVAL;
  if (cfg->head_dim != 128 && cfg->head_dim != 512) return KVC_EUNSUPPORTED;
  if (cfg->rope_dim < 0 || cfg->rope_dim > cfg->head_dim || cfg->rope_dim % 2 != 0) return KVC_EINVAL;
  if (cfg->x_format != KVC_X_F32 && cfg->x_format != KVC_X_BF16) return KVC_EINVAL;
  if (cfg->projection != KVC_PROJ_AUTO && cfg->projection != KVC_PROJ_BF16_SPLIT &&
      cfg->projection != KVC_PROJ_F32_MFMA && cfg->projection != KVC_PROJ_F16_SPLIT)
    return KVC_EINVAL;
  if ((cfg->projection == KVC_PROJ_F32_MFMA || cfg->projection == KVC_PROJ_F16_SPLIT) && cfg->x_format != KVC_X_F32)
    return KVC_EINVAL;
  return KVC_OK;
}

// the pooled compressor (ratio > 1)
int check_config(const kvc_config *cfg) {
  const int rc = check_common(cfg);
  if (rc) return rc;
  if (cfg->ratio != 2 && cfg->ratio != 4 && cfg->ratio != 128) return KVC_EUNSUPPORTED;
  return KVC_OK;
}

// the ratio-1 compressor
int check_ratio1(const kvc_config *cfg) {
  const int rc = check_common(cfg);
  if (rc) return rc;
  if (cfg->ratio != 1) return KVC_EINVAL;
  return cfg->rope_dim == 0 ? KVC_OK : KVC_EUNSUPPORTED;
}

bool overlapped(const kvc_config *cfg) { return cfg->ratio == 4; }
// the projection KVC_PROJ_AUTO stands for: the f32 matrix cores for f32
// rows, the exact bf16 split for bf16 rows (whose products with the three
// bf16 parts of the weights are exact)
int32_t projection_of(const kvc_config *cfg) {
  if (cfg->projection != KVC_PROJ_AUTO) return cfg->projection;
  return cfg->x_format == KVC_X_F32 ? KVC_PROJ_F32_MFMA : KVC_PROJ_BF16_SPLIT;
}
int64_t proj_of(const kvc_config *cfg) { return overlapped(cfg) ? 2 * (int64_t)cfg->head_dim : cfg->head_dim; }
int64_t rows_of(const kvc_config *cfg) { return overlapped(cfg) ? 2 * (int64_t)cfg->ratio : cfg->ratio; }

int check_projection_inputs(const kvc_config *cfg, const kvc_weights *w) {
  if (!w || !w->wkv || !w->wgate) return KVC_EINVAL;
  if (cfg->dim <= 0) return KVC_EINVAL;
  if (cfg->dim % 32 != 0 || cfg->dim > kMaxDim) return KVC_EUNSUPPORTED;
  if (!aligned(w->wkv) || !aligned(w->wgate)) return KVC_EINVAL;
  return KVC_OK;
}

int check_outputs(const kvc_config *cfg, const kvc_outputs *out) {
  if (!out) return KVC_OK;
  if (!aligned(out->latent) || !aligned(out->pooled) || !aligned(out->dequant) || !aligned(out->rotated))
    return KVC_EINVAL;
  if (out->rotated && cfg->rope_dim == 0) return KVC_EINVAL;
  // codes rows are head_dim / 2 bytes: 64 or 256, each lane stores up to 4
  if (out->codes && (reinterpret_cast<uintptr_t>(out->codes) % 4) != 0) return KVC_EINVAL;
  return KVC_OK;
}

bool wants_entries(const kvc_outputs *out) {
  return out && (out->latent || out->pooled || out->codes || out->scales || out->dequant || out->rotated);
}

// With RoPE, every entry written needs its table row: entries
// [first, first + count) of the sequence.
int check_rope(const kvc_config *cfg, const kvc_weights *w, int64_t first, int64_t count) {
  if (cfg->rope_dim == 0 || count <= 0) return KVC_OK;
  if (!w || !w->rope_cs || !aligned(w->rope_cs)) return KVC_EINVAL;
  return first + count <= w->rope_rows ? KVC_OK : KVC_EINVAL;
}

// Decode splits the K range over workgroups so that about 256 of them (one
// per CU) share the batch's projection: 32 columns x 64 rows per workgroup,
// at most 16 splits.
int32_t decode_splits(const kvc_config *cfg, int64_t batch) {
  const int64_t m_tiles = (batch + 63) / 64;
  const int64_t n_tiles = 2 * proj_of(cfg) / 32;
  const int64_t want = 256 / (m_tiles * n_tiles);
  int32_t s = 1;
  while (2 * s <= want && s < 16) s *= 2;
  return s;
}

int hip_status(hipError_t e) { return e == hipSuccess ? KVC_OK : KVC_EHIP; }

// Decode workspace: the partial sums (f32 x: the k segments, [kKSegments]
// [batch][2 proj]; bf16 x: the split-K parts, [splits][2][batch][proj]; given
// projections: [2][batch][proj] at the start), then the f32 path's arrival
// counters, one per tile, rounded up to 64.
int64_t decode_partial_floats(const kvc_config *cfg, int64_t batch) {
  const int64_t halves = kvc::kKSegments * 2 * batch * proj_of(cfg);
  const int32_t splits = cfg->dim > 0 && cfg->dim % 32 == 0 ? decode_splits(cfg, batch) : 1;
  const int64_t parts = (int64_t)splits * 2 * batch * proj_of(cfg);
  return halves > parts ? halves : parts;
}
int64_t decode_counter_floats(const kvc_config *cfg, int64_t batch) {
  return (kvc::decode_f32_tiles(batch, proj_of(cfg)) + 63) / 64 * 64;
}

// The measurement hook of kvc_time_next_projection: events pending for this
// thread's next compressor call, taken (and cleared) at its start.
thread_local hipEvent_t g_time_start = nullptr, g_time_stop = nullptr;
struct ProjectionTimer {
  hipEvent_t start, stop;
  ProjectionTimer() : start(g_time_start), stop(g_time_stop) { g_time_start = g_time_stop = nullptr; }
  int before(hipStream_t s) const { return start ? hip_status(hipEventRecord(start, s)) : KVC_OK; }
  int after(hipStream_t s) const { return stop ? hip_status(hipEventRecord(stop, s)) : KVC_OK; }
};

int decode_step(const kvc_config *cfg, const kvc_weights *w, const void *x, int64_t batch, int64_t start_pos,
                float *part, uint32_t *counters, float *kv_state, float *score_state, int64_t state_batch,
                const kvc_outputs *out, int32_t *emitted, const ProjectionTimer &timer, hipStream_t s);

// Prefill workspace: the kv and score planes, then (ratio 4) the f32 pooled
// entries of the fused projection + pooling path, then for the f32 matrix
// cores the running sums of a ragged last row tile (256 rows of both
// planes' columns), or the split weights: bf16 [2 proj][3][dim]
// (KVC_PROJ_BF16_SPLIT), or f16 [2 proj][2][dim] followed by the int32 scale
// exponents of the 2 proj weight rows and of the batch * seqlen rows of x
// (KVC_PROJ_F16_SPLIT; each part 16-byte aligned).
int64_t pooled_floats(const kvc_config *cfg, int64_t batch, int64_t seqlen) {
  return overlapped(cfg) ? batch * (seqlen / cfg->ratio) * cfg->head_dim : 0;
}
int64_t split_offset(const kvc_config *cfg, int64_t batch, int64_t seqlen) {
  return 2 * batch * seqlen * proj_of(cfg) + pooled_floats(cfg, batch, seqlen);
}
int64_t round4(int64_t v) { return (v + 3) / 4 * 4; }
int64_t split_floats(const kvc_config *cfg, int64_t m) {
  if (cfg->dim <= 0) return 0;
  switch (projection_of(cfg)) {
    case KVC_PROJ_F16_SPLIT: return 2 * proj_of(cfg) * cfg->dim + 2 * proj_of(cfg) + round4(m);
    case KVC_PROJ_BF16_SPLIT: return 3 * proj_of(cfg) * cfg->dim;
    default: return kvc::gemm_rag_floats(proj_of(cfg));  // the f32 matrix cores
  }
}

// The fused path (projection GEMM with pooling in its epilogue) needs 4-token
// blocks aligned with the flattened rows and enough 256 x 256 tiles to fill
// the chip twice; smaller problems run the GEMM and pool kernels separately.
bool use_fused_pooling(const kvc_config *cfg, int64_t batch, int64_t seqlen, int64_t workspace_floats) {
  if (!overlapped(cfg) || seqlen / cfg->ratio == 0) return false;
  if (batch > 1 && seqlen % 4 != 0) return false;
  const int64_t m = batch * seqlen;
  if (kvc::gemm_pool_row_tiles(m) * (cfg->head_dim / 64) < 512) return false;
  return workspace_floats >= 2 * m * proj_of(cfg) + pooled_floats(cfg, batch, seqlen);
}

kvc::PoolArgs pool_args(const kvc_config *cfg, const kvc_weights *w, const kvc_outputs *out) {
  kvc::PoolArgs p{};
  p.ape = w ? w->ape : nullptr;
  p.norm_w = w ? w->norm_w : nullptr;
  p.eps = cfg->eps;
  p.latent = out->latent;
  p.pooled = out->pooled;
  p.codes = out->codes;
  p.scales = out->scales;
  p.deq = out->dequant;
  p.e8m0 = cfg->fp4_format == KVC_FP4_E8M0_B32;
  // the table is read only when entries are written (its rows are checked then)
  p.rope_cs = (cfg->rope_dim > 0 && w && wants_entries(out)) ? w->rope_cs : nullptr;
  p.rope_dim = cfg->rope_dim;
  p.rope_row0 = 0;
  p.rotated = out->rotated;
  return p;
}

// Entries per wavefront run: one entry per wavefront up to 4096 entries
// (many short wavefronts keep the most loads in flight), then runs that
// keep about 4096 wavefronts (measured on gfx950 at 16384 entries of 512
// features: 4 entries per wavefront 0.785 of HBM peak, 1 entry 0.767).
int32_t entries_per_wave(int64_t batch, int64_t groups) {
  const int64_t total = batch * groups;
  int64_t e = (total + 4095) / 4096;
  if (e < 1) e = 1;
  if (e > 16) e = 16;
  return (int32_t)e;
}

}  // namespace

extern "C" {

int64_t kvc_proj_width(const kvc_config *cfg) {
  const int rc = check_config(cfg);
  return rc ? rc : proj_of(cfg);
}

int64_t kvc_state_rows(const kvc_config *cfg) {
  const int rc = check_config(cfg);
  return rc ? rc : rows_of(cfg);
}

int64_t kvc_prefill_workspace_floats(const kvc_config *cfg, int64_t batch, int64_t seqlen) {
  const int rc = check_config(cfg);
  if (rc) return rc;
  if (batch < 1 || seqlen < 0) return KVC_EINVAL;
  return split_offset(cfg, batch, seqlen) + split_floats(cfg, batch * seqlen);
}

int64_t kvc_decode_workspace_floats(const kvc_config *cfg, int64_t batch) {
  const int rc = check_config(cfg);
  if (rc) return rc;
  if (batch < 1) return KVC_EINVAL;
  return decode_partial_floats(cfg, batch) + decode_counter_floats(cfg, batch);
}

int kvc_time_next_projection(void *start, void *stop) {
  if ((start == nullptr) != (stop == nullptr)) return KVC_EINVAL;
  g_time_start = static_cast<hipEvent_t>(start);
  g_time_stop = static_cast<hipEvent_t>(stop);
  return KVC_OK;
}

int compressor_prefill(const kvc_config *cfg, const kvc_weights *w, const void *x, int64_t batch, int64_t seqlen,
                       float *workspace, int64_t workspace_floats, float *kv_state, float *score_state,
                       int64_t state_batch, const kvc_outputs *out, int64_t *n_groups, kvc_stream stream) {
  const ProjectionTimer timer;
  int rc = check_config(cfg);
  if (rc) return rc;
  if (batch < 1 || seqlen < 0) return KVC_EINVAL;
  if (x) {
    if ((rc = check_projection_inputs(cfg, w))) return rc;
    if (!aligned(x)) return KVC_EINVAL;
  }
  if (w && (!aligned(w->ape) || !aligned(w->norm_w))) return KVC_EINVAL;
  const int64_t proj = proj_of(cfg);
  const int64_t m = batch * seqlen;
  const bool x_bf16 = cfg->x_format == KVC_X_BF16;
  // with x the split weights sit after the planes and pooled rows
  const int32_t projection = projection_of(cfg);
  const bool with_x = x && m > 0;
  const int64_t need = with_x ? split_offset(cfg, batch, seqlen) + split_floats(cfg, m) : 2 * m * proj;
  if (need > 0 && !workspace) return KVC_EINVAL;
  if (workspace_floats < need) return KVC_ESPACE;
  if (!aligned(workspace)) return KVC_EINVAL;
  if ((kv_state == nullptr) != (score_state == nullptr)) return KVC_EINVAL;
  if (kv_state && (state_batch < batch || !aligned(kv_state) || !aligned(score_state))) return KVC_EINVAL;
  if ((rc = check_outputs(cfg, out))) return rc;

  const int64_t groups = seqlen / cfg->ratio;
  if (wants_entries(out) && (rc = check_rope(cfg, w, 0, groups))) return rc;
  if (n_groups) *n_groups = groups;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float *kv_plane = workspace;
  float *sc_plane = workspace ? workspace + m * proj : nullptr;

  const bool fused = x && m > 0 && wants_entries(out) && use_fused_pooling(cfg, batch, seqlen, workspace_floats);
  if (x && m > 0) {
    kvc::GemmArgs g{};
    g.a = x_bf16 ? nullptr : static_cast<const float *>(x);
    g.a16 = x_bf16 ? static_cast<const uint16_t *>(x) : nullptr;
    g.b0 = w->wkv;
    g.b1 = w->wgate;
    g.c0 = kv_plane;
    g.c1 = sc_plane;
    g.lda = cfg->dim;
    g.ldb = cfg->dim;
    g.ldc = proj;
    g.m = m;
    g.n_half = proj;
    g.k = cfg->dim;
    g.splits = 1;
    g.c_split_stride = 0;
    // the positional bias joins the gate logits in the GEMM epilogue
    g.bias1 = w->ape;
    g.bias_seqlen = seqlen;
    g.bias_ratio = cfg->ratio;
    if (fused) {
      g.pooled = workspace + 2 * m * proj;
      g.pool_batch = batch;
      g.pool_seqlen = seqlen;
      g.pool_groups = groups;
      g.pool_hd = cfg->head_dim;
    }
    if (projection == KVC_PROJ_F32_MFMA) {
      g.rag = workspace + split_offset(cfg, batch, seqlen);
      if ((rc = timer.before(s))) return rc;
      rc = hip_status(fused ? kvc::launch_gemm_pool(g, s) : kvc::launch_gemm(g, kvc::GemmShape::kPrefill, s));
      if (!rc) rc = timer.after(s);
    } else {
      // the weights' parts, in the row order the kernel reads
      const bool f16 = projection == KVC_PROJ_F16_SPLIT;
      float *split_base = workspace + split_offset(cfg, batch, seqlen);
      uint16_t *split = reinterpret_cast<uint16_t *>(split_base);
      int32_t *wexp = reinterpret_cast<int32_t *>(split_base + 2 * proj * cfg->dim);
      int32_t *xexp = wexp + 2 * proj;
      kvc::SplitArgs sa{};
      sa.w0 = w->wkv;
      sa.w1 = w->wgate;
      sa.ldw = cfg->dim;
      sa.n_half = proj;
      sa.k = cfg->dim;
      sa.pool_hd = fused ? cfg->head_dim : 0;
      // the column tile and wavefront columns of the kernel below
      sa.pool_tile = x_bf16 || f16 ? 256 : 128;
      sa.pool_wn = f16 ? 128 : 64;
      sa.out = split;
      sa.f16 = f16;
      sa.exp_out = f16 ? wexp : nullptr;
      if ((rc = hip_status(kvc::launch_split_weights(sa, s)))) return rc;
      g.bsplit = split;
      if (f16) {
        g.wexp = wexp;
        g.xexp = xexp;
        if ((rc = hip_status(kvc::launch_row_exponents(g.a, m, cfg->dim, cfg->dim, xexp, s)))) return rc;
      }
      if ((rc = timer.before(s))) return rc;
      if (f16) rc = hip_status(fused ? kvc::launch_gemm_h3_pool(g, s) : kvc::launch_gemm_h3(g, s));
      else if (x_bf16) rc = hip_status(fused ? kvc::launch_gemm_x3_pool(g, s) : kvc::launch_gemm_x3(g, s));
      else rc = hip_status(fused ? kvc::launch_gemm_x6_pool(g, s) : kvc::launch_gemm_x6(g, s));
      if (!rc) rc = timer.after(s);
    }
    if (rc) return rc;
  }
  // projections the caller put in the workspace carry no bias yet
  const float *ape_after = x ? nullptr : (w ? w->ape : nullptr);
  if (fused) {
    // pooled entries of the fused GEMM, then the row tiles' first entries,
    // then the per-entry epilogue over the pooled rows
    float *pooled = workspace + 2 * m * proj;
    kvc::PoolArgs pb{};
    pb.kv = kv_plane;
    pb.sc = sc_plane;
    pb.row_stride = proj;
    pb.batch_stride = seqlen * proj;
    pb.batch = batch;
    pb.groups = groups;
    pb.eps = cfg->eps;
    pb.pooled = pooled;
    pb.out_batch_stride = groups;
    if ((rc = hip_status(kvc::launch_pool_boundary(pb, kvc::gemm_pool_row_tiles(m), seqlen, cfg->head_dim, s))))
      return rc;
    kvc::PoolArgs pf = pool_args(cfg, w, out);
    pf.kv = pooled;
    pf.row_stride = cfg->head_dim;
    pf.batch = 1;
    pf.groups = batch * groups;
    pf.out_batch_stride = groups;
    if ((rc = hip_status(kvc::launch_rows_finish(pf, cfg->head_dim, s)))) return rc;
  } else if (groups > 0 && wants_entries(out)) {
    kvc::PoolArgs p = pool_args(cfg, w, out);
    p.ape = ape_after;
    p.kv = kv_plane;
    p.sc = sc_plane;
    p.row_stride = proj;
    p.batch_stride = seqlen * proj;
    p.batch = batch;
    p.groups = groups;
    p.first_entry = 0;
    p.entries_per_wave = entries_per_wave(batch, groups);
    p.out_batch_stride = groups;
    if ((rc = hip_status(kvc::launch_pool(p, cfg->ratio, cfg->head_dim, s)))) return rc;
  }
  if (kv_state) {
    kvc::StateStoreArgs st{};
    st.kv = kv_plane;
    st.sc = sc_plane;
    st.ape = ape_after;
    st.kv_state = kv_state;
    st.sc_state = score_state;
    st.batch = batch;
    st.seqlen = seqlen;
    st.proj = proj;
    st.state_rows = rows_of(cfg);
    st.ratio = cfg->ratio;
    st.overlap = overlapped(cfg);
    if ((rc = hip_status(kvc::launch_state_store(st, s)))) return rc;
  }
  return KVC_OK;
}

int compressor_decode_step(const kvc_config *cfg, const kvc_weights *w, const void *x, int64_t batch,
                           int64_t start_pos, float *workspace, int64_t workspace_floats, float *kv_state,
                           float *score_state, int64_t state_batch, const kvc_outputs *out, int32_t *emitted,
                           kvc_stream stream) {
  const ProjectionTimer timer;
  int rc = check_config(cfg);
  if (rc) return rc;
  if (batch < 1) return KVC_EINVAL;
  if (!workspace || !aligned(workspace)) return KVC_EINVAL;
  const int64_t part_floats = decode_partial_floats(cfg, batch);
  if (workspace_floats < part_floats + decode_counter_floats(cfg, batch)) return KVC_ESPACE;
  return decode_step(cfg, w, x, batch, start_pos, workspace, reinterpret_cast<uint32_t *>(workspace + part_floats),
                     kv_state, score_state, state_batch, out, emitted, timer, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace {

// One decode step with the partial sums in `part` (decode_partial_floats()
// floats; given projections at its start when x is NULL) and the f32 path's
// arrival counters in `counters` (decode_counter_floats(), zero at rest).
int decode_step(const kvc_config *cfg, const kvc_weights *w, const void *x, int64_t batch, int64_t start_pos,
                float *part, uint32_t *counters, float *kv_state, float *score_state, int64_t state_batch,
                const kvc_outputs *out, int32_t *emitted, const ProjectionTimer &timer, hipStream_t s) {
  int rc;
  if (batch < 1 || start_pos < 0) return KVC_EINVAL;
  if (x) {
    if ((rc = check_projection_inputs(cfg, w))) return rc;
    if (!aligned(x)) return KVC_EINVAL;
  }
  if (w && (!aligned(w->ape) || !aligned(w->norm_w))) return KVC_EINVAL;
  if (!kv_state || !score_state || state_batch < batch || !aligned(kv_state) || !aligned(score_state))
    return KVC_EINVAL;
  if ((rc = check_outputs(cfg, out))) return rc;

  const int r = cfg->ratio;
  const bool emit = start_pos > 0 && (start_pos + 1) % r == 0;
  // the emitted entry's index in the sequence (its RoPE table row)
  const int64_t entry = (start_pos + 1) / r - 1;
  if (emit && wants_entries(out) && (rc = check_rope(cfg, w, entry, 1))) return rc;
  if (emitted) *emitted = emit ? 1 : 0;
  const int64_t proj = proj_of(cfg);
  const int slot = (int)(start_pos % r);
  const int state_row = overlapped(cfg) ? r + slot : slot;
  const bool reset_prev = start_pos == 0 && overlapped(cfg);

  // the pooled entry of a completed group, over the state planes (whose
  // scores already hold the bias); at ratio 4 the block then shifts even
  // when no output is requested
  const bool pool_now = emit && (wants_entries(out) || overlapped(cfg));
  kvc::PoolArgs p = out ? pool_args(cfg, w, out) : kvc::PoolArgs{};
  p.ape = nullptr;
  p.norm_w = w ? w->norm_w : nullptr;
  p.eps = cfg->eps;
  p.kv = kv_state;
  p.sc = score_state;
  p.row_stride = proj;
  p.batch_stride = rows_of(cfg) * proj;
  p.batch = batch;
  p.groups = 1;
  p.first_entry = overlapped(cfg) ? 1 : 0;
  p.rope_row0 = entry;
  p.entries_per_wave = 1;
  p.out_batch_stride = 1;
  if (overlapped(cfg)) {
    p.shift_kv = kv_state;
    p.shift_sc = score_state;
  }

  if (x && cfg->x_format == KVC_X_F32) {
    // one launch: the projection (the prefill's two k halves) and the ingest
    kvc::DecodeArgs d{};
    d.x = static_cast<const float *>(x);
    d.w0 = w->wkv;
    d.w1 = w->wgate;
    d.m = batch;
    d.k = cfg->dim;
    d.n_half = proj;
    d.seg = kvc::kseg_length(cfg->dim);
    d.part = part;
    d.counters = counters;
    d.ape = w->ape;
    d.kv_state = kv_state;
    d.sc_state = score_state;
    d.state_rows = rows_of(cfg);
    d.slot = slot;
    d.state_row = state_row;
    d.reset_rows = reset_prev ? r : 0;
    if ((rc = timer.before(s))) return rc;
    if ((rc = hip_status(kvc::launch_decode_f32(d, s)))) return rc;
    if ((rc = timer.after(s))) return rc;
    // a group completed: pool it (the only other launch of the step)
    if (pool_now)
      return hip_status(overlapped(cfg) ? kvc::launch_decode_emit(p, cfg->head_dim, s)
                                        : kvc::launch_pool(p, r, cfg->head_dim, s));
    return KVC_OK;
  }

  // bf16 rows (split-K partials) or given projections: the projection, then
  // one launch that sums the parts, ingests and (groups of 2 and 4) pools
  const int32_t splits = x ? decode_splits(cfg, batch) : 1;
  if (x) {
    kvc::GemmArgs g{};
    g.a16 = static_cast<const uint16_t *>(x);
    g.b0 = w->wkv;
    g.b1 = w->wgate;
    g.c0 = part;
    g.c1 = part + batch * proj;
    g.lda = cfg->dim;
    g.ldb = cfg->dim;
    g.ldc = proj;
    g.m = batch;
    g.n_half = proj;
    g.k = cfg->dim;
    g.splits = splits;
    g.c_split_stride = 2 * batch * proj;
    if ((rc = timer.before(s))) return rc;
    if ((rc = hip_status(kvc::launch_gemm(g, kvc::GemmShape::kDecode, s)))) return rc;
    if ((rc = timer.after(s))) return rc;
  }
  kvc::IngestArgs in{};
  in.part = part;
  in.splits = splits;
  in.ape = w ? w->ape : nullptr;
  in.kv_state = kv_state;
  in.sc_state = score_state;
  in.batch = batch;
  in.proj = proj;
  in.state_rows = rows_of(cfg);
  in.slot = slot;
  in.state_row = state_row;
  in.ratio = r;
  in.reset_prev = reset_prev ? 1 : 0;
  if (pool_now && r != 128) {
    // ingest and pool in one launch
    return hip_status(kvc::launch_decode_finish(in, &p, cfg->head_dim, s));
  }
  if ((rc = hip_status(kvc::launch_decode_finish(in, nullptr, cfg->head_dim, s)))) return rc;
  if (pool_now && wants_entries(out)) {
    if ((rc = hip_status(kvc::launch_pool(p, r, cfg->head_dim, s)))) return rc;
  }
  return KVC_OK;
}

// The scratch of compressor_decode_step_noalloc: a file-scope device array
// (each GPU holds its own copy until the process ends), the partial sums
// first, then the arrival counters at a fixed place, so that they are zero
// at rest whatever the size of the previous call (device arrays start
// zeroed, and every completed step leaves the counters zero).
constexpr int64_t kScratchPartFloats = int64_t(1) << 20;  // 4 MiB of partial sums
constexpr int64_t kScratchCounterFloats = 4096;          // arrival counters
__device__ __align__(256) float scratch[kScratchPartFloats + kScratchCounterFloats];

// The device address of `scratch` on the current device, resolved once per
// device (host code must not pass the array's name to a kernel: in host
// code it stands for a host-side handle, not a device address).
constexpr int kMaxDevices = 64;
float *g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mutex;

int scratch_ptr(float **ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVC_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVC_EHIP;
    g_scratch_ptr[dev] = static_cast<float *>(p);
  }
  *ptr = g_scratch_ptr[dev];
  return KVC_OK;
}

}  // namespace

extern "C" {

int compressor_decode_step_noalloc(const kvc_config *cfg, const kvc_weights *w, const void *x, int64_t batch,
                                   int64_t start_pos, float *kv_state, float *score_state, int64_t state_batch,
                                   const kvc_outputs *out, int32_t *emitted, kvc_stream stream) {
  const ProjectionTimer timer;
  int rc = check_config(cfg);
  if (rc) return rc;
  if (batch < 1 || !x) return KVC_EINVAL;
  if (decode_partial_floats(cfg, batch) > kScratchPartFloats ||
      decode_counter_floats(cfg, batch) > kScratchCounterFloats)
    return KVC_ESPACE;
  float *base = nullptr;
  if ((rc = scratch_ptr(&base))) return rc;
  return decode_step(cfg, w, x, batch, start_pos, base, reinterpret_cast<uint32_t *>(base + kScratchPartFloats),
                     kv_state, score_state, state_batch, out, emitted, timer, reinterpret_cast<hipStream_t>(stream));
}

int64_t kvc_ratio1_workspace_floats(const kvc_config *cfg, int64_t tokens) {
  const int rc = check_ratio1(cfg);
  if (rc) return rc;
  if (tokens < 0) return KVC_EINVAL;
  return tokens * cfg->head_dim;
}

int compressor_ratio1_forward(const kvc_config *cfg, const uint16_t *wkv, const float *norm_w, const uint16_t *x,
                              int64_t tokens, float *workspace, int64_t workspace_floats, const kvc_outputs *out,
                              kvc_stream stream) {
  int rc = check_ratio1(cfg);
  if (rc) return rc;
  if (tokens < 0) return KVC_EINVAL;
  if (tokens == 0) return KVC_OK;
  if (!x || !wkv || !workspace) return KVC_EINVAL;
  if (cfg->dim <= 0) return KVC_EINVAL;
  if (cfg->dim % 64 != 0 || cfg->dim > kMaxDim) return KVC_EUNSUPPORTED;
  if (!aligned(x) || !aligned(wkv) || !aligned(norm_w) || !aligned(workspace)) return KVC_EINVAL;
  const int64_t hd = cfg->head_dim;
  if (workspace_floats < tokens * hd) return KVC_ESPACE;
  if ((rc = check_outputs(cfg, out))) return rc;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  kvc::GemmBf16Args g{};
  g.a = x;
  g.b = wkv;
  g.c = workspace;
  g.lda = cfg->dim;
  g.ldb = cfg->dim;
  g.ldc = hd;
  g.m = tokens;
  g.n = hd;
  g.k = cfg->dim;
  if ((rc = hip_status(kvc::launch_gemm_bf16(g, s)))) return rc;
  if (wants_entries(out)) {
    kvc::PoolArgs p = pool_args(cfg, nullptr, out);
    p.norm_w = norm_w;
    p.kv = workspace;
    p.row_stride = hd;
    p.batch_stride = tokens * hd;
    p.batch = 1;
    p.groups = tokens;
    p.out_batch_stride = tokens;
    if ((rc = hip_status(kvc::launch_rows_finish(p, cfg->head_dim, s)))) return rc;
  }
  return KVC_OK;
}

namespace {
int fp4_quant(const uint16_t *in, int64_t rows, int64_t width, uint8_t *codes, uint8_t *scales, uint16_t *out,
              int block, kvc_stream stream) {
  if (rows < 0 || width <= 0 || width % block != 0) return KVC_EINVAL;
  if (rows > 0 && !in) return KVC_EINVAL;
  if (!aligned(in) || !aligned(out) || (codes && reinterpret_cast<uintptr_t>(codes) % 4 != 0))
    return KVC_EINVAL;
  if (out && out != in) {
    // overlapping but distinct buffers would race
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(in), a1 = a0 + rows * width * 2;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(out), b1 = b0 + rows * width * 2;
    if (a0 < b1 && b0 < a1) return KVC_EINVAL;
  }
  return hip_status(kvc::launch_fp4_quant(in, rows, width, codes, scales, out, block == 32,
                                          reinterpret_cast<hipStream_t>(stream)));
}
}  // namespace

int latent_fp4_quant(const uint16_t *in, int64_t rows, int64_t width, uint8_t *codes, uint8_t *scales,
                     uint16_t *out, kvc_stream stream) {
  return fp4_quant(in, rows, width, codes, scales, out, 16, stream);
}

int indexer_fp4_quant(const uint16_t *in, int64_t rows, int64_t width, uint8_t *codes, uint8_t *scales,
                      uint16_t *out, kvc_stream stream) {
  return fp4_quant(in, rows, width, codes, scales, out, 32, stream);
}

int latent_rope(const uint16_t *in, int64_t rows, int64_t width, int32_t rope_dim, const float *rope_cs,
                int64_t rope_rows, int64_t first_row, uint16_t *out, kvc_stream stream) {
  if (rows < 0 || width <= 0 || width % 2 != 0 || rope_dim <= 0 || rope_dim % 2 != 0 || rope_dim > width)
    return KVC_EINVAL;
  if (rows == 0) return KVC_OK;
  if (!in || !out || !rope_cs || first_row < 0 || first_row + rows > rope_rows) return KVC_EINVAL;
  // 4-byte pairs and 8-byte (cos, sin) loads
  if (reinterpret_cast<uintptr_t>(in) % 4 || reinterpret_cast<uintptr_t>(out) % 4 ||
      reinterpret_cast<uintptr_t>(rope_cs) % 8)
    return KVC_EINVAL;
  if (out != in) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(in), a1 = a0 + rows * width * 2;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(out), b1 = b0 + rows * width * 2;
    if (a0 < b1 && b0 < a1) return KVC_EINVAL;
  }
  kvc::RopeArgs a{in, out, rows, width, rope_dim, rope_cs, first_row};
  return hip_status(kvc::launch_rope(a, reinterpret_cast<hipStream_t>(stream)));
}

const char *kvc_strerror(int code) {
  switch (code) {
    case KVC_OK: return "ok";
    case KVC_EINVAL: return "invalid argument (null pointer, size out of range or misaligned pointer)";
    case KVC_EUNSUPPORTED: return "unsupported configuration";
    case KVC_ESPACE: return "buffer too small";
    case KVC_EHIP: return "HIP launch failed";
    default: return "unknown error code";
  }
}

const char *kvc_version(void) { return "kvc 0.1.0 gfx950"; }

}  // extern "C"
