// Block plan for the frame-structured mask ("HeyGen x Google Cloud:
// Bringing Avatar IV to TPUs", section "Deleting the Mask", Fig. 3).
//
// Query frame f sees the key frames of the clamped window
// [f - window_before, f + window_after] plus the reference frames (ref_count
// consecutive frames from ref_frame); with ref_queries_global the reference
// frames' own queries see every frame. With block sizes that are multiples
// of 16 dividing the frame span, a (query block,
// key block) pair is live exactly when the key block's frame is live for
// the query block's frame, and then every token pair in it is live. So the
// plan is a frame-level list expanded to blocks: each query block of frame
// f lists the key blocks of its live frames, ascending.
#include <algorithm>
#include <climits>
#include <cstring>

#include "fsattn.h"
#include "fsattn_internal.h"

namespace fsattn {

bool geometry_ok(const fsattn_mask *m) {
  if (!m) return false;
  const int64_t F = m->num_frames, T = m->tokens_per_frame;
  if (F < 1 || T < 16 || T % 16 != 0) return false;
  if (F * T > INT32_MAX) return false;
  if (m->window_before < 0 || m->window_after < 0) return false;
  if (m->ref_frame < -1 || m->ref_frame >= F) return false;
  if (m->ref_queries_global != 0 && m->ref_queries_global != 1) return false;
  if (m->ref_count < 0) return false;
  if (m->ref_frame >= 0 && (int64_t)m->ref_frame + std::max(1, m->ref_count) > F) return false;
  for (int64_t b : {(int64_t)m->block_q, (int64_t)m->block_k})
    if (b <= 0 || b % 16 != 0 || T % b != 0) return false;
  return true;
}

int64_t live_frame_count(const fsattn_mask *m, int f) {
  int iv[4];
  const int n = live_intervals(live_geom(*m), f, iv);
  int64_t c = 0;
  for (int i = 0; i < n; ++i) c += iv[2 * i + 1] - iv[2 * i] + 1;
  return c;
}

int live_frames(const fsattn_mask *m, int f, int *out, int cap) {
  int iv[4];
  const int n = live_intervals(live_geom(*m), f, iv);
  int c = 0;
  for (int i = 0; i < n; ++i)
    for (int g = iv[2 * i]; g <= iv[2 * i + 1]; ++g, ++c)
      if (c < cap) out[c] = g;
  return c;
}

int max_runs_per_frame(const fsattn_mask *m) {
  // The window is one contiguous frame range; the span of reference frames
  // adds a second run unless it overlaps or touches the window.
  const LiveGeom g = live_geom(*m);
  int best = 0, iv[4];
  for (int f = 0; f < m->num_frames; ++f) best = std::max(best, live_intervals(g, f, iv));
  return best;
}

}  // namespace fsattn

using namespace fsattn;

extern "C" fsattn_status fsattn_plan_size(const fsattn_mask *m, int64_t *num_q_blocks, int64_t *nnz) {
  if (!m || !num_q_blocks || !nnz) return FSATTN_ERR_INVALID_ARGUMENT;
  if (!geometry_ok(m)) return FSATTN_ERR_BLOCK_GEOMETRY;
  const int64_t T = m->tokens_per_frame;
  const int64_t qpf = T / m->block_q, kpf = T / m->block_k;
  int64_t total = 0;
  for (int f = 0; f < m->num_frames; ++f) total += live_frame_count(m, f) * qpf * kpf;
  *num_q_blocks = (int64_t)m->num_frames * qpf;
  *nnz = total;
  return FSATTN_OK;
}

extern "C" fsattn_status fsattn_plan(const fsattn_mask *m, int32_t *row_ptr, int64_t row_ptr_len,
                                     int32_t *col_idx, int64_t col_idx_len) {
  if (!m || !row_ptr || (!col_idx && col_idx_len > 0)) return FSATTN_ERR_INVALID_ARGUMENT;
  int64_t nqb = 0, nnz = 0;
  fsattn_status st = fsattn_plan_size(m, &nqb, &nnz);
  if (st != FSATTN_OK) return st;
  if (nnz > INT32_MAX) return FSATTN_ERR_UNSUPPORTED;
  if (row_ptr_len < nqb + 1 || col_idx_len < nnz) return FSATTN_ERR_BUFFER_TOO_SMALL;
  const int T = m->tokens_per_frame;
  const int qpf = T / m->block_q, kpf = T / m->block_k;
  const LiveGeom g = live_geom(*m);
  int64_t pos = 0;
  int64_t qb = 0;
  row_ptr[0] = 0;
  for (int f = 0; f < m->num_frames; ++f) {
    int iv[4];
    const int n = live_intervals(g, f, iv);
    for (int i = 0; i < qpf; ++i) {
      // the live frames' key blocks, ascending: each interval of frames is
      // one contiguous range of key blocks
      for (int j = 0; j < n; ++j)
        for (int64_t c = (int64_t)iv[2 * j] * kpf; c < (int64_t)(iv[2 * j + 1] + 1) * kpf; ++c)
          col_idx[pos++] = (int32_t)c;
      row_ptr[++qb] = (int32_t)pos;
    }
  }
  return FSATTN_OK;
}
