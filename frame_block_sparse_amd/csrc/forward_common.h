// Device helpers shared by the forward kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <climits>

#include "fsattn_internal.h"

namespace fsattn {

// Turns a query block's list of live key blocks (a CSR row of the plan)
// into maximal runs of consecutive key blocks, as key-token ranges
// [x, y). The frame mask gives at most two runs per query frame (the window
// and, when it is not adjacent, the reference frame), so the kernels' inner
// loop walks contiguous key ranges and never tests a mask. Run by one wave;
// results land in LDS. Every index read is clamped to the plan arrays and
// every run to [0, N), so any plan contents stay in bounds.
__device__ inline void build_runs(const int32_t *row_ptr, const int32_t *col_idx, int64_t nnz,
                                  int qb, int bk, int N, int2 *runs, int *nruns) {
  const int lane = threadIdx.x & 63;
  int64_t base = row_ptr[qb];
  int64_t end = row_ptr[qb + 1];
  if (base < 0) base = 0;
  if (end > nnz) end = nnz;
  const int64_t cnt = end > base ? end - base : 0;
  int ns = 0, ne = 0;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t off = 0; off < cnt; off += 64) {
    const int64_t i = off + lane;
    const bool valid = i < cnt;
    const int c = valid ? col_idx[base + i] : 0;
    const int prev = (valid && i > 0) ? col_idx[base + i - 1] : INT_MIN;
    const int next = (valid && i + 1 < cnt) ? col_idx[base + i + 1] : INT_MIN;
    const bool st = valid && (i == 0 || prev == INT_MIN || c != prev + 1);
    const bool en = valid && (i + 1 == cnt || next == INT_MIN || next != c + 1);
    const unsigned long long sm = __ballot(st);
    const unsigned long long em = __ballot(en);
    const int rs = ns + __popcll(sm & below);
    const int re = ne + __popcll(em & below);
    const int64_t tok0 = (int64_t)c * bk, tok1 = ((int64_t)c + 1) * bk;
    if (st && rs < kMaxRuns) runs[rs].x = (int)min<int64_t>(max<int64_t>(tok0, 0), N);
    if (en && re < kMaxRuns) runs[re].y = (int)min<int64_t>(max<int64_t>(tok1, 0), N);
    ns += __popcll(sm);
    ne += __popcll(em);
  }
  if (lane == 0) *nruns = ns < kMaxRuns ? ns : kMaxRuns;
}

}  // namespace fsattn
