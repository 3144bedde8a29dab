// C entry points: argument validation, workspace layout and dispatch.
// Every check runs on the host before any launch; on error nothing is
// launched and no output is written.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "fsattn.h"
#include "fsattn_internal.h"

using namespace fsattn;

namespace {

// Tokens per bounds-kernel workgroup (within one frame): 128, or 256 for
// frames of 4096 tokens or more, where halving the chunk partial sums that
// the per-head kernel adds up outweighs the fewer workgroups (measured on
// 8160-token frames: 8 % less time; equal at 3600, slower at 960).
int bounds_chunk(int tokens_per_frame) { return tokens_per_frame >= 4096 ? 256 : 128; }

int elem_size(int dtype) { return dtype == FSATTN_BF16 ? 2 : 4; }

fsattn_status check_shape(const fsattn_shape *s, const fsattn_mask *m) {
  if (!s || !m) return FSATTN_ERR_INVALID_ARGUMENT;
  if (!geometry_ok(m)) return FSATTN_ERR_BLOCK_GEOMETRY;
  if (s->batch < 1 || s->heads < 1) return FSATTN_ERR_INVALID_ARGUMENT;
  if ((int64_t)s->seq_len != (int64_t)m->num_frames * m->tokens_per_frame) return FSATTN_ERR_INVALID_ARGUMENT;
  if (s->head_dim != 64 && s->head_dim != 128) return FSATTN_ERR_UNSUPPORTED;
  if (s->dtype != FSATTN_F32 && s->dtype != FSATTN_BF16) return FSATTN_ERR_UNSUPPORTED;
  if ((int64_t)s->batch * s->heads > 65535) return FSATTN_ERR_UNSUPPORTED;
  return FSATTN_OK;
}

fsattn_status check_tensor(const fsattn_tensor &t, int esz, int head_dim) {
  if (!t.data) return FSATTN_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(t.data) % 16) return FSATTN_ERR_INVALID_ARGUMENT;
  if (t.stride_b < 0 || t.stride_h < 0 || t.stride_n < head_dim) return FSATTN_ERR_INVALID_ARGUMENT;
  if ((t.stride_b * esz) % 16 || (t.stride_h * esz) % 16 || (t.stride_n * esz) % 16)
    return FSATTN_ERR_INVALID_ARGUMENT;
  return FSATTN_OK;
}

struct WsLayout {
  size_t part, frame, qmax, kmax, total;
  int chunk, chunks_per_frame;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

WsLayout ws_layout(const fsattn_shape *s, const fsattn_mask *m) {
  WsLayout w;
  const int64_t BH = (int64_t)s->batch * s->heads;
  w.chunk = bounds_chunk(m->tokens_per_frame);
  w.chunks_per_frame = (m->tokens_per_frame + w.chunk - 1) / w.chunk;
  const int64_t NC = (int64_t)m->num_frames * w.chunks_per_frame;
  const int64_t D = s->head_dim;
  size_t off = 0;
  w.part = off;  off = align256(off + sizeof(float) * BH * NC * D);
  w.frame = off; off = align256(off + sizeof(float) * BH * m->num_frames * D);
  w.qmax = off;  off = align256(off + sizeof(float) * BH * NC);
  w.kmax = off;  off = align256(off + sizeof(float) * BH * NC);
  w.total = off;
  return w;
}

BoundsParams bounds_params(const fsattn_shape *s, const fsattn_mask *m, const fsattn_tensor &q,
                           const fsattn_tensor &k, float scale, float gap_threshold_nats, float *key_mean,
                           fsattn_head_bound *rec, void *workspace, const WsLayout &w) {
  BoundsParams p;
  p.q = q.data; p.k = k.data;
  p.qsb = q.stride_b; p.qsh = q.stride_h; p.qsn = q.stride_n;
  p.ksb = k.stride_b; p.ksh = k.stride_h; p.ksn = k.stride_n;
  p.B = s->batch; p.H = s->heads; p.N = s->seq_len; p.F = m->num_frames; p.T = m->tokens_per_frame;
  p.D = s->head_dim;
  p.live = live_geom(*m);
  p.chunk = w.chunk; p.chunks_per_frame = w.chunks_per_frame;
  p.scale = scale; p.threshold = gap_threshold_nats;
  p.key_mean = key_mean; p.rec = rec;
  char *base = static_cast<char *>(workspace);
  p.ws_part = reinterpret_cast<float *>(base + w.part);
  p.ws_frame = reinterpret_cast<float *>(base + w.frame);
  p.ws_qmax = reinterpret_cast<float *>(base + w.qmax);
  p.ws_kmax = reinterpret_cast<float *>(base + w.kmax);
  return p;
}

}  // namespace

extern "C" int fsattn_abi_version(void) { return FSATTN_ABI_VERSION; }

extern "C" const char *fsattn_status_string(fsattn_status st) {
  switch (st) {
    case FSATTN_OK: return "ok";
    case FSATTN_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FSATTN_ERR_BLOCK_GEOMETRY:
      return "block sizes must be positive multiples of 16 dividing tokens_per_frame";
    case FSATTN_ERR_UNSUPPORTED: return "unsupported head_dim, dtype or launch shape";
    case FSATTN_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case FSATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

extern "C" fsattn_status fsattn_plan_device(void *hip_stream, const fsattn_mask *m, int32_t *row_ptr,
                                            int64_t row_ptr_len, int32_t *col_idx, int64_t col_idx_len) {
  if (!m || !row_ptr || (!col_idx && col_idx_len > 0)) return FSATTN_ERR_INVALID_ARGUMENT;
  int64_t nqb = 0, nnz = 0;
  fsattn_status st = fsattn_plan_size(m, &nqb, &nnz);
  if (st != FSATTN_OK) return st;
  if (nnz > INT32_MAX) return FSATTN_ERR_UNSUPPORTED;
  if (row_ptr_len < nqb + 1 || col_idx_len < nnz) return FSATTN_ERR_BUFFER_TOO_SMALL;
  const hipError_t e = launch_plan_device(*m, row_ptr, col_idx, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? FSATTN_OK : FSATTN_ERR_HIP;
}

extern "C" size_t fsattn_head_bounds_workspace_bytes(const fsattn_shape *s, const fsattn_mask *m) {
  if (check_shape(s, m) != FSATTN_OK) return 0;
  return ws_layout(s, m).total;
}

extern "C" fsattn_status fsattn_head_bounds(void *hip_stream, const fsattn_shape *s, const fsattn_mask *m,
                                            fsattn_tensor q, fsattn_tensor k, float scale,
                                            float gap_threshold_nats, float *key_mean,
                                            fsattn_head_bound *rec, void *workspace,
                                            size_t workspace_bytes) {
  fsattn_status st = check_shape(s, m);
  if (st != FSATTN_OK) return st;
  const int esz = elem_size(s->dtype);
  if ((st = check_tensor(q, esz, s->head_dim)) != FSATTN_OK) return st;
  if ((st = check_tensor(k, esz, s->head_dim)) != FSATTN_OK) return st;
  if (!(scale > 0.f) || !std::isfinite(scale)) return FSATTN_ERR_INVALID_ARGUMENT;
  if (!(gap_threshold_nats >= 0.f)) return FSATTN_ERR_INVALID_ARGUMENT;
  if (!key_mean || !rec || !workspace) return FSATTN_ERR_INVALID_ARGUMENT;
  const WsLayout w = ws_layout(s, m);
  if (workspace_bytes < w.total) return FSATTN_ERR_BUFFER_TOO_SMALL;
  const BoundsParams p = bounds_params(s, m, q, k, scale, gap_threshold_nats, key_mean, rec, workspace, w);
  const hipError_t e = launch_head_bounds(p, s->dtype, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? FSATTN_OK : FSATTN_ERR_HIP;
}

extern "C" fsattn_status fsattn_head_bounds_noalloc(void *hip_stream, const fsattn_shape *s,
                                                    const fsattn_mask *m, fsattn_tensor q, fsattn_tensor k,
                                                    float scale, float gap_threshold_nats, float *key_mean,
                                                    fsattn_head_bound *rec) {
  fsattn_status st = check_shape(s, m);
  if (st != FSATTN_OK) return st;
  const int esz = elem_size(s->dtype);
  if ((st = check_tensor(q, esz, s->head_dim)) != FSATTN_OK) return st;
  if ((st = check_tensor(k, esz, s->head_dim)) != FSATTN_OK) return st;
  if (!(scale > 0.f) || !std::isfinite(scale)) return FSATTN_ERR_INVALID_ARGUMENT;
  if (!(gap_threshold_nats >= 0.f)) return FSATTN_ERR_INVALID_ARGUMENT;
  if (!key_mean || !rec) return FSATTN_ERR_INVALID_ARGUMENT;
  const WsLayout w = ws_layout(s, m);
  if (w.total > kBoundsScratchBytes) return FSATTN_ERR_BUFFER_TOO_SMALL;
  void *scratch = nullptr;
  if (bounds_scratch(&scratch) != hipSuccess) return FSATTN_ERR_HIP;
  const BoundsParams p = bounds_params(s, m, q, k, scale, gap_threshold_nats, key_mean, rec, scratch, w);
  const hipError_t e = launch_head_bounds(p, s->dtype, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? FSATTN_OK : FSATTN_ERR_HIP;
}

extern "C" size_t fsattn_head_bounds_noalloc_max_workspace(void) { return kBoundsScratchBytes; }

extern "C" fsattn_status fsattn_produce(void *hip_stream, const fsattn_shape *s, const fsattn_mask *m,
                                        fsattn_tensor q_in, fsattn_tensor k_in, fsattn_tensor v_in,
                                        const float *gamma_q, const float *gamma_k, float eps,
                                        const float *rope_cos, const float *rope_sin, fsattn_tensor q,
                                        fsattn_tensor k, fsattn_tensor v, float scale,
                                        float gap_threshold_nats, float *key_mean, fsattn_head_bound *rec,
                                        void *workspace, size_t workspace_bytes) {
  fsattn_status st = check_shape(s, m);
  if (st != FSATTN_OK) return st;
  const int esz = elem_size(s->dtype);
  for (const fsattn_tensor *t : {&q_in, &k_in, &v_in, &q, &k, &v})
    if ((st = check_tensor(*t, esz, s->head_dim)) != FSATTN_OK) return st;
  if (!(scale > 0.f) || !std::isfinite(scale)) return FSATTN_ERR_INVALID_ARGUMENT;
  if (!(gap_threshold_nats >= 0.f)) return FSATTN_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return FSATTN_ERR_INVALID_ARGUMENT;
  if (!key_mean || !rec || !workspace) return FSATTN_ERR_INVALID_ARGUMENT;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return FSATTN_ERR_INVALID_ARGUMENT;
  for (const float *g : {gamma_q, gamma_k, rope_cos, rope_sin})
    if (reinterpret_cast<uintptr_t>(g) % 16) return FSATTN_ERR_INVALID_ARGUMENT;
  const WsLayout w = ws_layout(s, m);
  if (workspace_bytes < w.total) return FSATTN_ERR_BUFFER_TOO_SMALL;
  const BoundsParams p = bounds_params(s, m, q, k, scale, gap_threshold_nats, key_mean, rec, workspace, w);
  ProduceParams x;
  x.qi = q_in.data; x.ki = k_in.data; x.vi = v_in.data;
  x.qisb = q_in.stride_b; x.qish = q_in.stride_h; x.qisn = q_in.stride_n;
  x.kisb = k_in.stride_b; x.kish = k_in.stride_h; x.kisn = k_in.stride_n;
  x.visb = v_in.stride_b; x.vish = v_in.stride_h; x.visn = v_in.stride_n;
  x.qo = q.data; x.ko = k.data;   // read back by the bounds through p.q, p.k (same strides)
  x.vo = v.data; x.vosb = v.stride_b; x.vosh = v.stride_h; x.vosn = v.stride_n;
  x.gq = gamma_q; x.gk = gamma_k; x.rcos = rope_cos; x.rsin = rope_sin;
  x.eps = eps;
  const hipError_t e = launch_produce(p, x, s->dtype, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? FSATTN_OK : FSATTN_ERR_HIP;
}

namespace {

constexpr uint32_t kKnownFlags = 0x7u | (0xfu << 8) | (0xfu << 12) | (0xfu << 16) | (0xfu << 20) | (0xfu << 24);

fsattn_status check_forward_host(const fsattn_shape *s, const fsattn_mask *m, uint32_t flags, FwdConfig *cfg) {
  fsattn_status st = check_shape(s, m);
  if (st != FSATTN_OK) return st;
  if (flags & ~kKnownFlags) return FSATTN_ERR_INVALID_ARGUMENT;
  if ((flags & 3) == 3) return FSATTN_ERR_INVALID_ARGUMENT;
  // the bf16 kernel walks at most two key runs per query frame (window and
  // reference frame), which is all this mask family produces
  if (max_runs_per_frame(m) > (s->dtype == FSATTN_BF16 ? 2 : kMaxRuns)) return FSATTN_ERR_UNSUPPORTED;
  if (s->dtype == FSATTN_F32 && (flags & (0xfffffu << 8))) return FSATTN_ERR_UNSUPPORTED;
  if (!choose_fwd_config(s, m, flags, cfg)) return FSATTN_ERR_UNSUPPORTED;
  if (cfg->grid / ((int64_t)s->batch * s->heads) > INT32_MAX) return FSATTN_ERR_UNSUPPORTED;
  // the bf16 grid covers every tile plus at most kXcds - 1 idle ids
  if (s->dtype == FSATTN_BF16 && cfg->grid > INT32_MAX - kXcds) return FSATTN_ERR_UNSUPPORTED;
  return FSATTN_OK;
}

}  // namespace

extern "C" fsattn_status fsattn_forward_launch_info(const fsattn_shape *s, const fsattn_mask *m, uint32_t flags,
                                                    int32_t *waves, int32_t *rows_per_wave, int32_t *key_step,
                                                    int64_t *workgroups, int32_t *lds_bytes) {
  FwdConfig c;
  const fsattn_status st = check_forward_host(s, m, flags, &c);
  if (st != FSATTN_OK) return st;
  if (waves) *waves = c.waves;
  if (rows_per_wave) *rows_per_wave = 16 * c.m16;
  if (key_step) *key_step = 16 * c.nk16;
  if (workgroups) *workgroups = c.grid;
  if (lds_bytes) *lds_bytes = c.lds_bytes;
  return FSATTN_OK;
}

extern "C" fsattn_status fsattn_forward(void *hip_stream, const fsattn_shape *s, const fsattn_mask *m,
                                        const int32_t *row_ptr, const int32_t *col_idx, int64_t nnz,
                                        fsattn_tensor q, fsattn_tensor k, fsattn_tensor v, fsattn_tensor o,
                                        int32_t o_dtype, const float *key_mean, const fsattn_head_bound *rec,
                                        float scale, uint32_t flags, float *lse) {
  FwdConfig cfg;
  fsattn_status st = check_forward_host(s, m, flags, &cfg);
  if (st != FSATTN_OK) return st;
  const int esz = elem_size(s->dtype);
  if ((st = check_tensor(q, esz, s->head_dim)) != FSATTN_OK) return st;
  if ((st = check_tensor(k, esz, s->head_dim)) != FSATTN_OK) return st;
  if ((st = check_tensor(v, esz, s->head_dim)) != FSATTN_OK) return st;
  if (o_dtype != s->dtype && o_dtype != FSATTN_F32) return FSATTN_ERR_UNSUPPORTED;
  if ((st = check_tensor(o, elem_size(o_dtype), s->head_dim)) != FSATTN_OK) return st;
  if (!row_ptr || !col_idx) return FSATTN_ERR_INVALID_ARGUMENT;
  // the bf16 kernel addresses one staged step (at most 64 rows) with 32-bit
  // byte offsets from the step's first row
  if (s->dtype == FSATTN_BF16 &&
      (k.stride_n * esz * 64 >= ((int64_t)1 << 31) || v.stride_n * esz * 64 >= ((int64_t)1 << 31)))
    return FSATTN_ERR_UNSUPPORTED;
  int64_t nqb = 0, want_nnz = 0;
  if ((st = fsattn_plan_size(m, &nqb, &want_nnz)) != FSATTN_OK) return st;
  if (nnz != want_nnz) return FSATTN_ERR_INVALID_ARGUMENT;
  const int mode = flags & 3;
  if (mode != FSATTN_MODE_FORCE_ONLINE && (!key_mean || !rec)) return FSATTN_ERR_INVALID_ARGUMENT;
  if (key_mean && reinterpret_cast<uintptr_t>(key_mean) % 16) return FSATTN_ERR_INVALID_ARGUMENT;
  if (!(scale > 0.f) || !std::isfinite(scale)) return FSATTN_ERR_INVALID_ARGUMENT;

  FwdParams p;
  p.q = q.data; p.k = k.data; p.v = v.data; p.o = o.data;
  p.qsb = q.stride_b; p.qsh = q.stride_h; p.qsn = q.stride_n;
  p.ksb = k.stride_b; p.ksh = k.stride_h; p.ksn = k.stride_n;
  p.vsb = v.stride_b; p.vsh = v.stride_h; p.vsn = v.stride_n;
  p.osb = o.stride_b; p.osh = o.stride_h; p.osn = o.stride_n;
  p.row_ptr = row_ptr; p.col_idx = col_idx; p.nnz = nnz;
  p.key_mean = key_mean; p.rec = rec; p.lse = lse;
  p.B = s->batch; p.H = s->heads; p.N = s->seq_len; p.F = m->num_frames; p.T = m->tokens_per_frame;
  p.bq = m->block_q; p.bk = m->block_k;
  p.wb = m->window_before; p.wa = m->window_after; p.ref = m->ref_frame;
  p.prior_pass = 0; p.tiles128 = 0; p.part_o = p.part_lse = nullptr;
  p.scale = scale; p.scale_log2 = scale * kLog2e;
  p.flags = flags;
  p.o_f32 = o_dtype == FSATTN_F32 ? 1 : 0;
  // heavy frames (most live key frames) first; ties keep frame order
  p.ordered = frame_issue_order(m, p.frame_order) ? 1 : 0;
  p.deal_chunk = 1;
  const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e;
  if (s->dtype == FSATTN_F32) {
    p.rows_per_wg = f32_rows_per_wg(p.T);
    p.tiles_per_frame = p.T / p.rows_per_wg;
    e = launch_forward_f32(p, s->head_dim, stream);
  } else {
    p.rows_per_wg = 16 * cfg.m16 * cfg.waves;
    p.tiles_per_frame = (p.T + p.rows_per_wg - 1) / p.rows_per_wg;
    p.deal_chunk = choose_deal_chunk(s, m, cfg, (int)((flags >> 24) & 15));
    // XCD x runs ids x, x + kXcds, ...: as many ids per XCD as the longest list
    int64_t longest = 0;
    for (int x = 0; x < kXcds; ++x) longest = std::max(longest, xcd_tile_count(cfg.grid, p.deal_chunk, x));
    cfg.grid = kXcds * longest;
    e = launch_forward_bf16(p, cfg, s->head_dim, stream);
  }
  return e == hipSuccess ? FSATTN_OK : FSATTN_ERR_HIP;
}

extern "C" fsattn_status fsattn_mfma_probe(void *hip_stream, int32_t workgroups, int32_t iters, float *sink,
                                           int64_t *flops) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || !sink) return FSATTN_ERR_INVALID_ARGUMENT;
  if (flops) *flops = mfma_probe_flops(workgroups, iters);
  const hipError_t e = launch_mfma_probe(workgroups, iters, sink, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? FSATTN_OK : FSATTN_ERR_HIP;
}

namespace {

struct PriorLayout {
  size_t o_w, lse_w, o_r, lse_r, total;
};

PriorLayout prior_layout(const fsattn_shape *s) {
  const int64_t rows = (int64_t)s->batch * s->heads * s->seq_len;
  PriorLayout l;
  size_t off = 0;
  l.o_w = off;   off = align256(off + sizeof(float) * rows * s->head_dim);
  l.lse_w = off; off = align256(off + sizeof(float) * rows);
  l.o_r = off;   off = align256(off + sizeof(float) * rows * s->head_dim);
  l.lse_r = off; off = align256(off + sizeof(float) * rows);
  l.total = off;
  return l;
}

}  // namespace

extern "C" size_t fsattn_prior_art_workspace_bytes(const fsattn_shape *s, const fsattn_mask *m) {
  if (check_shape(s, m) != FSATTN_OK || s->dtype != FSATTN_BF16) return 0;
  return prior_layout(s).total;
}

extern "C" fsattn_status fsattn_prior_art_forward(void *hip_stream, const fsattn_shape *s, const fsattn_mask *m,
                                                  fsattn_tensor q, fsattn_tensor k, fsattn_tensor v,
                                                  fsattn_tensor o, int32_t o_dtype, float scale, void *workspace,
                                                  size_t workspace_bytes) {
  fsattn_status st = check_shape(s, m);
  if (st != FSATTN_OK) return st;
  if (s->dtype != FSATTN_BF16) return FSATTN_ERR_UNSUPPORTED;
  if (m->ref_frame >= 0 && (m->ref_queries_global || m->ref_count > 1)) return FSATTN_ERR_UNSUPPORTED;
  const int esz = elem_size(s->dtype);
  if ((st = check_tensor(q, esz, s->head_dim)) != FSATTN_OK) return st;
  if ((st = check_tensor(k, esz, s->head_dim)) != FSATTN_OK) return st;
  if ((st = check_tensor(v, esz, s->head_dim)) != FSATTN_OK) return st;
  if (o_dtype != s->dtype && o_dtype != FSATTN_F32) return FSATTN_ERR_UNSUPPORTED;
  if ((st = check_tensor(o, elem_size(o_dtype), s->head_dim)) != FSATTN_OK) return st;
  if (k.stride_n * esz * 64 >= ((int64_t)1 << 31) || v.stride_n * esz * 64 >= ((int64_t)1 << 31))
    return FSATTN_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return FSATTN_ERR_INVALID_ARGUMENT;
  if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 16) return FSATTN_ERR_INVALID_ARGUMENT;
  const PriorLayout l = prior_layout(s);
  if (workspace_bytes < l.total) return FSATTN_ERR_BUFFER_TOO_SMALL;
  const int64_t tiles = ((int64_t)s->seq_len + 127) / 128;
  if (tiles * s->batch * s->heads > INT32_MAX) return FSATTN_ERR_UNSUPPORTED;

  FwdParams p = {};
  p.q = q.data; p.k = k.data; p.v = v.data; p.o = o.data;
  p.qsb = q.stride_b; p.qsh = q.stride_h; p.qsn = q.stride_n;
  p.ksb = k.stride_b; p.ksh = k.stride_h; p.ksn = k.stride_n;
  p.vsb = v.stride_b; p.vsh = v.stride_h; p.vsn = v.stride_n;
  p.osb = o.stride_b; p.osh = o.stride_h; p.osn = o.stride_n;
  p.B = s->batch; p.H = s->heads; p.N = s->seq_len; p.F = m->num_frames; p.T = m->tokens_per_frame;
  p.bq = m->block_q; p.bk = m->block_k;
  p.wb = m->window_before; p.wa = m->window_after; p.ref = m->ref_frame;
  p.scale = scale; p.scale_log2 = scale * kLog2e;
  p.flags = FSATTN_MODE_FORCE_ONLINE;
  p.o_f32 = o_dtype == FSATTN_F32 ? 1 : 0;
  p.rows_per_wg = 128;
  p.tiles128 = (int)tiles;
  char *base = static_cast<char *>(workspace);
  float *o_w = reinterpret_cast<float *>(base + l.o_w), *lse_w = reinterpret_cast<float *>(base + l.lse_w);
  float *o_r = reinterpret_cast<float *>(base + l.o_r), *lse_r = reinterpret_cast<float *>(base + l.lse_r);
  const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  // pass 0: the window; pass 1: the reference frame, for rows whose window
  // does not hold it; then the merge
  p.prior_pass = 0; p.part_o = o_w; p.part_lse = lse_w;
  hipError_t e = launch_prior_pass_bf16(p, s->head_dim, stream);
  const bool has_ref = m->ref_frame >= 0;
  if (e == hipSuccess && has_ref) {
    p.prior_pass = 1; p.part_o = o_r; p.part_lse = lse_r;
    e = launch_prior_pass_bf16(p, s->head_dim, stream);
  }
  if (e == hipSuccess)
    e = launch_prior_merge(o_w, lse_w, has_ref ? o_r : nullptr, lse_r, p.B, p.H, p.N, s->head_dim, o.data,
                           p.o_f32, o.stride_b, o.stride_h, o.stride_n, stream);
  return e == hipSuccess ? FSATTN_OK : FSATTN_ERR_HIP;
}
