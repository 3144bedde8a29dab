// Block plan written on the GPU ("HeyGen x Google Cloud: Bringing Avatar IV
// to TPUs", section "Deleting the Mask", Fig. 3): the same CSR arrays as the
// host plan, element for element, straight into device memory.
//
// Query frame f sees the key frames of the clamped window
// [f - window_before, f + window_after] plus the reference frame (all frames
// for a global reference frame's own queries), so every
// query block of frame f lists the same key blocks: those of its live
// frames, ascending. One workgroup per query frame finds where the frame's
// rows start (the sum of the earlier frames' row lengths), then writes its
// row_ptr entries and its col_idx rows with consecutive threads on
// consecutive entries.
#include <hip/hip_runtime.h>

#include "fsattn_internal.h"

namespace fsattn {
namespace {

constexpr int kPlanThreads = 256;

struct PlanGeom {
  int F, wb, wa, ref, ref_global, qpf, kpf;
};

// Live frames of query frame f: the clamped window [lo, hi], plus the
// reference frame before (extra = -1) or after (extra = +1) it, or none
// (extra = 0) when there is no reference frame or it lies in the window.
__device__ inline void live_of(const PlanGeom &g, int f, int &lo, int &hi, int &extra) {
  const bool all = g.ref_global && f == g.ref;
  const int64_t l = (int64_t)f - g.wb, h = (int64_t)f + g.wa;   // (windows may be wider than F)
  lo = all || l < 0 ? 0 : (int)l;
  hi = all || h > g.F - 1 ? g.F - 1 : (int)h;
  extra = 0;
  if (g.ref >= 0 && g.ref < lo) extra = -1;
  if (g.ref >= 0 && g.ref > hi) extra = 1;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanGeom g, int32_t *row_ptr, int32_t *col_idx) {
  __shared__ int64_t part[kPlanThreads];
  const int f = blockIdx.x;
  const int t = threadIdx.x;
  // entries before frame f: its predecessors' live-frame counts times the
  // blocks per frame pair
  int64_t before = 0;
  for (int h = t; h < f; h += kPlanThreads) {
    int lo, hi, extra;
    live_of(g, h, lo, hi, extra);
    before += (int64_t)(hi - lo + 1 + (extra != 0));
  }
  part[t] = before;
  __syncthreads();
  for (int o = kPlanThreads / 2; o > 0; o >>= 1) {
    if (t < o) part[t] += part[t + o];
    __syncthreads();
  }
  const int64_t base = part[0] * g.qpf * g.kpf;
  int lo, hi, extra;
  live_of(g, f, lo, hi, extra);
  const int n = hi - lo + 1 + (extra != 0);
  const int E = n * g.kpf;   // entries per query block of this frame
  if (f == 0 && t == 0) row_ptr[0] = 0;
  for (int i = t; i < g.qpf; i += kPlanThreads)
    row_ptr[(int64_t)f * g.qpf + i + 1] = (int32_t)(base + (int64_t)(i + 1) * E);
  const int64_t total = (int64_t)g.qpf * E;
  for (int64_t idx = t; idx < total; idx += kPlanThreads) {
    const int e = (int)(idx % E);
    const int j = e / g.kpf, c = e % g.kpf;   // j-th live frame, its c-th key block
    int frame;
    if (extra < 0) frame = j == 0 ? g.ref : lo + j - 1;
    else if (extra > 0) frame = j == n - 1 ? g.ref : lo + j;
    else frame = lo + j;
    col_idx[base + idx] = frame * g.kpf + c;
  }
}

}  // namespace

hipError_t launch_plan_device(const fsattn_mask &m, int32_t *row_ptr, int32_t *col_idx, hipStream_t st) {
  PlanGeom g;
  g.F = m.num_frames;
  g.wb = m.window_before;
  g.wa = m.window_after;
  g.ref = m.ref_frame;
  g.ref_global = m.ref_queries_global;
  g.qpf = m.tokens_per_frame / m.block_q;
  g.kpf = m.tokens_per_frame / m.block_k;
  hipLaunchKernelGGL(plan_kernel, dim3(g.F), dim3(kPlanThreads), 0, st, g, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace fsattn
