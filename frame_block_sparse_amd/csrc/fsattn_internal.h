// Internal declarations shared by the host layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "fsattn.h"

namespace fsattn {

constexpr int kMaxRuns = 64;        // contiguous key runs per query frame kept in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// The mask's frame geometry as the kernels see it: the window, and the
// reference frames r .. r + nr - 1 (nr = 0 without reference frames), whose
// own queries see every frame when rg is set.
struct LiveGeom {
  int F, wb, wa, r, nr, rg;
};

inline LiveGeom live_geom(const fsattn_mask &m) {
  LiveGeom g;
  g.F = m.num_frames;
  g.wb = m.window_before;
  g.wa = m.window_after;
  g.r = m.ref_frame;
  g.nr = m.ref_frame >= 0 ? (m.ref_count > 1 ? m.ref_count : 1) : 0;
  g.rg = m.ref_frame >= 0 ? m.ref_queries_global : 0;
  return g;
}

// The frames whose keys the queries of frame f see, as one or two disjoint,
// non-adjacent intervals in ascending order: [iv[0], iv[1]] and, when two
// are returned, [iv[2], iv[3]]. The window [f - wb, f + wa] is clamped to
// [0, F - 1]; the span of reference frames is merged into it when they
// overlap or touch.
__host__ __device__ inline int live_intervals(const LiveGeom &g, int f, int iv[4]) {
  if (g.rg && f >= g.r && f < g.r + g.nr) {
    iv[0] = 0;
    iv[1] = g.F - 1;
    return 1;
  }
  const int64_t l = (int64_t)f - g.wb, h = (int64_t)f + g.wa;   // (windows may be wider than F)
  const int lo = l < 0 ? 0 : (int)l, hi = h > g.F - 1 ? g.F - 1 : (int)h;
  iv[0] = lo;
  iv[1] = hi;
  if (g.nr == 0) return 1;
  const int ra = g.r, rb = g.r + g.nr - 1;
  if (ra <= hi + 1 && rb >= lo - 1) {
    iv[0] = ra < lo ? ra : lo;
    iv[1] = rb > hi ? rb : hi;
    return 1;
  }
  if (rb < lo) {
    iv[0] = ra; iv[1] = rb; iv[2] = lo; iv[3] = hi;
  } else {
    iv[2] = ra; iv[3] = rb;
  }
  return 2;
}

// Host-side geometry helpers (fsattn_plan.cpp).
bool geometry_ok(const fsattn_mask *m);
// Live frames of query frame f in ascending order; returns the count.
int live_frames(const fsattn_mask *m, int f, int *out, int cap);
int64_t live_frame_count(const fsattn_mask *m, int f);
// Largest number of contiguous key-frame runs over all query frames.
int max_runs_per_frame(const fsattn_mask *m);

struct BoundsParams {
  const void *q, *k;
  int64_t qsb, qsh, qsn, ksb, ksh, ksn;
  int B, H, N, F, T, D;
  LiveGeom live;                 // window and reference frames
  int chunk, chunks_per_frame;  // token chunk (within one frame)
  float scale, threshold;
  float *key_mean;
  fsattn_head_bound *rec;
  float *ws_part;     // [BH][NC][D] partial key sums
  float *ws_frame;    // [BH][F][D]  per-frame key sums
  float *ws_qmax;     // [BH][NC]    partial max |q|^2
  float *ws_kmax;     // [BH][NC]    partial max |k - mu|^2
};

hipError_t launch_head_bounds(const BoundsParams &p, int dtype, hipStream_t st);

// The device-resident workspace of fsattn_head_bounds_noalloc: its size,
// and its address on the current device (bounds_kernels.hip).
constexpr size_t kBoundsScratchBytes = size_t(4) << 20;
constexpr int kMaxDevices = 64;
hipError_t bounds_scratch(void **ptr);

// The input-producing chain fused into the bounds' first pass
// (fsattn_produce): Q, K and V are read through the input views, Q and K are
// RMS-normalised (gamma [H][d], when given) and rotated (angle tables
// [N][d/2], when given), and all three are written through the output
// views qo, ko, vo; qo and ko are the views BoundsParams' q and k then read
// (same pointers and strides).
struct ProduceParams {
  const void *qi, *ki, *vi;
  int64_t qisb, qish, qisn, kisb, kish, kisn, visb, vish, visn;
  void *qo, *ko, *vo;
  int64_t vosb, vosh, vosn;
  const float *gq, *gk;         // [H][d] or null (no normalisation)
  const float *rcos, *rsin;     // [N][d/2] or null (no rotation)
  float eps;
};
hipError_t launch_produce(const BoundsParams &p, const ProduceParams &x, int dtype, hipStream_t st);

// Device plan (same arrays as fsattn_plan); the mask is already validated.
hipError_t launch_plan_device(const fsattn_mask &m, int32_t *row_ptr, int32_t *col_idx, hipStream_t st);

struct FwdParams {
  const void *q, *k, *v;
  void *o;
  int64_t qsb, qsh, qsn, ksb, ksh, ksn, vsb, vsh, vsn, osb, osh, osn;
  const int32_t *row_ptr, *col_idx;
  int64_t nnz;
  const float *key_mean;
  const fsattn_head_bound *rec;
  float *lse;
  int B, H, N, F, T, bq, bk;
  int rows_per_wg, tiles_per_frame;
  float scale, scale_log2;
  uint32_t flags;
  int o_f32;
  // Frames in the order their workgroups are issued (most live frames first);
  // used when num_frames <= kMaxOrderedFrames, natural order otherwise.
  int ordered;
  uint8_t frame_order[64];
  // Tiles per chunk dealt to one XCD (see dealt_tile).
  int deal_chunk;
  // Prior-art comparator (tiled passes, see fsattn_prior_art_forward): the
  // pass (0 window, 1 reference frame), query tiles of 128 rows, and the
  // pass's normalised fp32 rows [B*H][N][d] and log-sum-exps [B*H][N].
  int prior_pass, tiles128;
  int wb, wa, ref;   // the mask's window and reference frame
  float *part_o, *part_lse;
};
constexpr int kMaxOrderedFrames = 64;

// The hardware deals workgroup ids round-robin over the XCDs of the device,
// so XCD x runs ids x, x + kXcds, ... in order.
constexpr int kXcds = 8;

// The forward's G query tiles in issue order (heaviest frames first, the
// tiles of one (frame, head) group consecutive) are cut into chunks of C
// tiles, and the chunks are dealt round-robin to the XCDs; the tiles of a
// last, partial round are shared out in contiguous ranges. Tile t of XCD x's
// list is tile dealt_tile(G, C, x, t) of the issue order; the lists' lengths
// differ by at most one.
__host__ __device__ inline int64_t xcd_tile_count(int64_t G, int64_t C, int x) {
  const int64_t A = G / (kXcds * C), Rt = G - kXcds * A * C;
  return A * C + ((x + 1) * Rt / kXcds - x * Rt / kXcds);
}
__host__ __device__ inline int64_t dealt_tile(int64_t G, int64_t C, int x, int64_t t) {
  const int64_t A = G / (kXcds * C);
  if (t < A * C) return (kXcds * (t / C) + x) * C + t % C;
  const int64_t Rt = G - kXcds * A * C;
  return kXcds * A * C + x * Rt / kXcds + (t - A * C);
}

struct FwdConfig {
  int waves, m16, nk16, nbuf;   // waves per workgroup, rows per wave / 16, keys per step / 16, ring buffers
  int lds_bytes;
  int64_t grid;
};

// Chooses (or validates an override of) the launch shape; false if none fits.
bool choose_fwd_config(const fsattn_shape *s, const fsattn_mask *m, uint32_t flags, FwdConfig *cfg);
hipError_t launch_forward_bf16(const FwdParams &p, const FwdConfig &c, int head_dim, hipStream_t st);
// Workgroups of this launch shape resident per CU on the current device (0
// if unknown).
int fwd_bf16_occupancy(const FwdConfig &c, int head_dim);
// Issue order of the query frames, heaviest first (fsattn_schedule.cpp);
// false when the natural order is used (more than kMaxOrderedFrames frames).
bool frame_issue_order(const fsattn_mask *m, uint8_t *order);
// Chunk size of the dealing (fsattn_schedule.cpp): `override` 0 picks it
// from a model of the per-XCD dispatch on the current device, 1..14 give
// 2^(override-1) tiles, 15 whole (frame, head) groups. Host only.
int choose_deal_chunk(const fsattn_shape *s, const fsattn_mask *m, const FwdConfig &c, int override);
hipError_t launch_forward_f32(const FwdParams &p, int head_dim, hipStream_t st);
// Prior-art comparator: one tiled pass of the bf16 forward kernel, and the
// merge of the two passes' rows into O (forward_bf16.hip).
hipError_t launch_prior_pass_bf16(const FwdParams &p, int head_dim, hipStream_t st);
hipError_t launch_prior_merge(const float *o_w, const float *lse_w, const float *o_r, const float *lse_r,
                              int B, int H, int N, int D, void *o, int o_f32, int64_t osb, int64_t osh,
                              int64_t osn, hipStream_t st);
// Pure-MFMA reference loop (mfma_probe.hip) and the FLOPs one launch does.
hipError_t launch_mfma_probe(int workgroups, int iters, float *sink, hipStream_t st);
int64_t mfma_probe_flops(int workgroups, int iters);
int f32_rows_per_wg(int T);

}  // namespace fsattn
