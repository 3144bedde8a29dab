// Block plan written on the GPU ("HeyGen x Google Cloud: Bringing Avatar IV
// to TPUs", section "Deleting the Mask", Fig. 3): the same CSR arrays as the
// host plan, element for element, straight into device memory.
//
// Query frame f sees the key frames of the clamped window
// [f - window_before, f + window_after] plus the reference frames (all
// frames for the queries of global reference frames), so every
// query block of frame f lists the same key blocks: those of its live
// frames, ascending. The query blocks of a frame are split over several
// workgroups (blockIdx.y); each finds where the frame's rows start (the sum
// of the earlier frames' row lengths), writes the row_ptr entries of its
// query blocks, and writes their col_idx rows: a thread computes the
// column of row entry e once and stores it into every row of its slice,
// consecutive threads on consecutive entries.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "fsattn_internal.h"

namespace fsattn {
namespace {

constexpr int kPlanThreads = 256;

struct PlanGeom {
  LiveGeom live;
  int qpf, kpf;
  int qb_per_wg;   // query blocks per workgroup
};

// Number of frames in the live intervals of query frame f.
__device__ inline int live_count(const LiveGeom &g, int f, int iv[4], int *first) {
  const int n = live_intervals(g, f, iv);
  *first = iv[1] - iv[0] + 1;
  return n == 1 ? *first : *first + iv[3] - iv[2] + 1;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanGeom g, int32_t *row_ptr, int32_t *col_idx) {
  __shared__ int64_t part[kPlanThreads];
  const int f = blockIdx.x;
  const int t = threadIdx.x;
  // this workgroup's query blocks of frame f
  const int q0 = blockIdx.y * g.qb_per_wg, q1 = min(g.qpf, q0 + g.qb_per_wg);
  // entries before frame f: its predecessors' live-frame counts times the
  // blocks per frame pair
  int64_t before = 0;
  for (int h = t; h < f; h += kPlanThreads) {
    int iv[4], first;
    before += live_count(g.live, h, iv, &first);
  }
  part[t] = before;
  __syncthreads();
  for (int o = kPlanThreads / 2; o > 0; o >>= 1) {
    if (t < o) part[t] += part[t + o];
    __syncthreads();
  }
  const int64_t base = part[0] * g.qpf * g.kpf;
  int iv[4], first;
  const int n = live_count(g.live, f, iv, &first);
  const int E = n * g.kpf;   // entries per query block of this frame
  if (f == 0 && q0 == 0 && t == 0) row_ptr[0] = 0;
  for (int i = q0 + t; i < q1; i += kPlanThreads)
    row_ptr[(int64_t)f * g.qpf + i + 1] = (int32_t)(base + (int64_t)(i + 1) * E);
  for (int e = t; e < E; e += kPlanThreads) {
    const int j = e / g.kpf, c = e % g.kpf;   // j-th live frame, its c-th key block
    const int frame = j < first ? iv[0] + j : iv[2] + (j - first);
    const int32_t col = frame * g.kpf + c;
    for (int i = q0; i < q1; ++i) col_idx[base + (int64_t)i * E + e] = col;
  }
}

}  // namespace

hipError_t launch_plan_device(const fsattn_mask &m, int32_t *row_ptr, int32_t *col_idx, hipStream_t st) {
  PlanGeom g;
  g.live = live_geom(m);
  g.qpf = m.tokens_per_frame / m.block_q;
  g.kpf = m.tokens_per_frame / m.block_k;
  // about 256 workgroups in all (the frames' query blocks split evenly)
  const int slices = std::max(1, std::min(g.qpf, (256 + g.live.F - 1) / g.live.F));
  g.qb_per_wg = (g.qpf + slices - 1) / slices;
  const int ny = (g.qpf + g.qb_per_wg - 1) / g.qb_per_wg;
  hipLaunchKernelGGL(plan_kernel, dim3(g.live.F, ny), dim3(kPlanThreads), 0, st, g, row_ptr, col_idx);
  return hipGetLastError();
}

}  // namespace fsattn
