// Block plan for the frame-structured mask ("HeyGen x Google Cloud:
// Bringing Avatar IV to TPUs", section "Deleting the Mask", Fig. 3).
//
// Query frame f sees the key frames of the clamped window
// [f - window_before, f + window_after] plus the reference frame; with
// ref_queries_global the reference frame's own queries see every frame.
// With block sizes that are multiples of 16 dividing the frame span, a (query block,
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
  for (int64_t b : {(int64_t)m->block_q, (int64_t)m->block_k})
    if (b <= 0 || b % 16 != 0 || T % b != 0) return false;
  return true;
}

static void window_of(const fsattn_mask *m, int f, int *lo, int *hi) {
  if (m->ref_queries_global && m->ref_frame >= 0 && f == m->ref_frame) {
    *lo = 0;   // a global reference frame's queries see every frame
    *hi = m->num_frames - 1;
    return;
  }
  const int64_t l = std::max<int64_t>(0, (int64_t)f - m->window_before);
  const int64_t h = std::min<int64_t>((int64_t)m->num_frames - 1, (int64_t)f + m->window_after);
  *lo = (int)l;
  *hi = (int)h;
}

int64_t live_frame_count(const fsattn_mask *m, int f) {
  int lo, hi;
  window_of(m, f, &lo, &hi);
  int64_t n = hi - lo + 1;
  if (m->ref_frame >= 0 && (m->ref_frame < lo || m->ref_frame > hi)) n += 1;
  return n;
}

int live_frames(const fsattn_mask *m, int f, int *out, int cap) {
  int lo, hi;
  window_of(m, f, &lo, &hi);
  const int r = m->ref_frame;
  int n = 0;
  auto put = [&](int x) { if (n < cap) out[n] = x; n++; };
  if (r >= 0 && r < lo) put(r);
  for (int g = lo; g <= hi; ++g) put(g);
  if (r >= 0 && r > hi) put(r);
  return n;
}

int max_runs_per_frame(const fsattn_mask *m) {
  // The window is one contiguous frame range; the reference frame adds a
  // second run unless it is inside or adjacent to the window.
  int best = 0;
  for (int f = 0; f < m->num_frames; ++f) {
    int lo, hi;
    window_of(m, f, &lo, &hi);
    const int r = m->ref_frame;
    int runs = 1;
    if (r >= 0 && (r < lo - 1 || r > hi + 1)) runs = 2;
    best = std::max(best, runs);
  }
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
  int frames[4096];
  int64_t pos = 0;
  int64_t qb = 0;
  row_ptr[0] = 0;
  for (int f = 0; f < m->num_frames; ++f) {
    const int n = live_frames(m, f, frames, 4096);
    for (int i = 0; i < qpf; ++i) {
      if (n <= 4096) {
        for (int j = 0; j < n; ++j)
          for (int c = 0; c < kpf; ++c) col_idx[pos++] = frames[j] * kpf + c;
      } else {  // very wide windows: enumerate frames directly, same order
        int lo, hi;
        window_of(m, f, &lo, &hi);
        const int r = m->ref_frame;
        auto emit = [&](int g) { for (int c = 0; c < kpf; ++c) col_idx[pos++] = g * kpf + c; };
        if (r >= 0 && r < lo) emit(r);
        for (int g = lo; g <= hi; ++g) emit(g);
        if (r >= 0 && r > hi) emit(r);
      }
      row_ptr[++qb] = (int32_t)pos;
    }
  }
  return FSATTN_OK;
}
