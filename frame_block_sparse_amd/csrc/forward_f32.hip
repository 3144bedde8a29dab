// fp32 forward: frame-block-sparse attention computed in fp32 throughout
// (products, exponentials, accumulation), for fp32 inputs where the result
// must stay within 1e-5 of exact softmax attention.
//
// One 64-lane workgroup per tile of R query rows (R a multiple of 16
// dividing the frame span, at most 64), one row per lane. Keys stream
// through LDS 16 at a time along the contiguous runs of the plan; every
// lane reads the same key (an LDS broadcast). The softmax uses either the
// per-row fixed shift of "Unchaining the Softmax" (bound plus scale*q.mu)
// or the online running max, chosen per head.
#include <hip/hip_runtime.h>

#include "forward_common.h"

namespace fsattn {
namespace {

template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdParams p) {
  __shared__ __align__(16) float ks[16][D];
  __shared__ __align__(16) float vs[16][D];
  __shared__ int2 runs[kMaxRuns];
  __shared__ int nruns;
  const int tile = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.H, h = bh % p.H;
  const int f = tile / p.tiles_per_frame, ti = tile % p.tiles_per_frame;
  const int row0 = f * p.T + ti * p.rows_per_wg;
  const int i = threadIdx.x;
  build_runs(p.row_ptr, p.col_idx, p.nnz, row0 / p.bq, p.bk, p.N, runs, &nruns);

  const float *qrow = static_cast<const float *>(p.q) + b * p.qsb + h * p.qsh;
  const float *kb = static_cast<const float *>(p.k) + b * p.ksb + h * p.ksh;
  const float *vb = static_cast<const float *>(p.v) + b * p.vsb + h * p.vsh;
  const bool active = i < p.rows_per_wg;
  const int row = row0 + (active ? i : 0);
  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    const float4 x = *reinterpret_cast<const float4 *>(qrow + (int64_t)row * p.qsn + d);
    q[d] = x.x; q[d + 1] = x.y; q[d + 2] = x.z; q[d + 3] = x.w;
    acc[d] = acc[d + 1] = acc[d + 2] = acc[d + 3] = 0.f;
  }
  const int mode = p.flags & 3;
  const bool fixed = mode == FSATTN_MODE_FORCE_FIXED ||
                     (mode == FSATTN_MODE_AUTO && p.rec[bh].eligible != 0);
  float shift;   // log2 units
  if (fixed) {
    const float *mu = p.key_mean + (int64_t)bh * D;
    float dot = 0.f, nq = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      dot = fmaf(q[d], mu[d], dot);
      nq = fmaf(q[d], q[d], nq);
    }
    const float m = (p.flags & FSATTN_SHIFT_PER_ROW)
                        ? p.scale * (sqrtf(nq) * p.rec[bh].k_norm_max + dot)
                        : p.rec[bh].bound + p.scale * dot;
    shift = m * kLog2e;
  } else {
    shift = -INFINITY;
  }
  float lsum = 0.f;
  __syncthreads();
  const int nr = nruns;
  for (int r = 0; r < nr; ++r) {
    const int k0 = runs[r].x, k1 = runs[r].y;
    for (int ks0 = k0; ks0 < k1; ks0 += 16) {
      const int kl = min(16, k1 - ks0);
      __syncthreads();
      for (int u = i; u < 16 * (D / 4); u += 64) {
        const int rr = u / (D / 4), c = (u % (D / 4)) * 4;
        if (rr < kl) {
          *reinterpret_cast<float4 *>(&ks[rr][c]) =
              *reinterpret_cast<const float4 *>(kb + (int64_t)(ks0 + rr) * p.ksn + c);
          *reinterpret_cast<float4 *>(&vs[rr][c]) =
              *reinterpret_cast<const float4 *>(vb + (int64_t)(ks0 + rr) * p.vsn + c);
        }
      }
      __syncthreads();
      float s[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float a = 0.f;
        if (j < kl) {
#pragma unroll
          for (int d = 0; d < D; ++d) a = fmaf(q[d], ks[j][d], a);
        }
        s[j] = j < kl ? a * p.scale_log2 : -INFINITY;
      }
      if (!fixed) {
        float mx = s[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mx = fmaxf(mx, s[j]);
        const float mn = fmaxf(shift, mx);
        const float alpha = exp2f(shift - mn);
        lsum *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] *= alpha;
        shift = mn;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j < kl) {
          const float e = exp2f(s[j] - shift);
          lsum += e;
#pragma unroll
          for (int d = 0; d < D; ++d) acc[d] = fmaf(e, vs[j][d], acc[d]);
        }
      }
    }
  }
  if (!active) return;
  const float inv = 1.f / lsum;
  float *orow = static_cast<float *>(p.o) + b * p.osb + h * p.osh + (int64_t)row * p.osn;
#pragma unroll
  for (int d = 0; d < D; d += 4)
    *reinterpret_cast<float4 *>(orow + d) =
        make_float4(acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv);
  if (p.lse) p.lse[(int64_t)bh * p.N + row] = (shift + log2f(lsum)) * kLn2;
}

}  // namespace

int f32_rows_per_wg(int T) {
  for (int r = 64; r >= 16; r -= 16)
    if (T % r == 0) return r;
  return 16;
}

hipError_t launch_forward_f32(const FwdParams &p, int head_dim, hipStream_t st) {
  const dim3 grid(p.F * p.tiles_per_frame, p.B * p.H);
  if (head_dim == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(64), 0, st, p);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(64), 0, st, p);
  return hipGetLastError();
}

}  // namespace fsattn
