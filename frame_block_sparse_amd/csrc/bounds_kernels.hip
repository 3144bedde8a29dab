// Per-head bound record ("HeyGen x Google Cloud: Bringing Avatar IV to
// TPUs", section "Unchaining the Softmax"): key mean, query-norm maximum,
// mean-centred key-norm maximum, the Cauchy-Schwarz logit bound, the window
// term c_max of the bound audit for windowed masks, and eligibility.
//
// Four launches; the two passes stream Q and K (HBM-bound), the other two
// are small:
//   pass1   per (token chunk, head): partial key sums, partial max |q|^2
//   frames  per (frame, head): the frame's key sum from its chunks
//   pass2   per (token chunk, head): key mean from the frame sums, partial
//           max |k - mu|^2
//   final   per head: max |q|, max |k - mu|, c_max from the frame sums,
//           bound, gap estimate, eligibility
// Chunks never cross a frame, so the per-frame sums are sums of whole
// chunks. Every reduction has a fixed order and no atomics are used, so the
// results are bitwise reproducible run to run.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include "fsattn_internal.h"

namespace fsattn {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ inline void load8(const T *p, float *x);

template <>
__device__ inline void load8<float>(const float *p, float *x) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  const float4 b = *reinterpret_cast<const float4 *>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <>
__device__ inline void load8<__hip_bfloat16>(const __hip_bfloat16 *p, float *x) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Sum over the `width` consecutive lanes that hold one token row.
__device__ inline float row_sum(float v, int width) {
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ inline float block_max(float v, float *sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if (t < o) sh[t] = fmaxf(sh[t], sh[t + o]);
    __syncthreads();
  }
  const float r = sh[0];
  __syncthreads();
  return r;
}

// sum_{i < n} x[i * stride], added in index order, with up to 8 loads in
// flight (the order of the additions is the plain sequential one).
__device__ inline float ordered_sum(const float *x, int n, int64_t stride) {
  float s = 0.f;
  int i = 0;
  for (; i + 8 <= n; i += 8) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = x[(int64_t)(i + e) * stride];
#pragma unroll
    for (int e = 0; e < 8; ++e) s += v[e];
  }
  for (; i < n; ++i) s += x[(int64_t)i * stride];
  return s;
}

// Token range [t0, t1) of chunk `c` (frame-major; chunks stay inside a frame).
__device__ inline void chunk_range(const BoundsParams &p, int c, int *t0, int *t1) {
  const int f = c / p.chunks_per_frame, ci = c % p.chunks_per_frame;
  *t0 = f * p.T + ci * p.chunk;
  *t1 = min(*t0 + p.chunk, (f + 1) * p.T);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bounds_pass1(BoundsParams p) {
  constexpr int TPR = D / 8;            // threads per token row (8 elements each)
  constexpr int RPP = kThreads / TPR;   // rows per pass
  __shared__ float sh[RPP][D + 1];
  __shared__ float red[kThreads];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.H, h = bh % p.H;
  const int NC = p.F * p.chunks_per_frame;
  const int col = threadIdx.x % TPR, r = threadIdx.x / TPR;
  const T *q = static_cast<const T *>(p.q) + b * p.qsb + h * p.qsh + col * 8;
  const T *k = static_cast<const T *>(p.k) + b * p.ksb + h * p.ksh + col * 8;
  int t0, t1;
  chunk_range(p, c, &t0, &t1);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float qm = 0.f;
  for (int t = t0 + r; t < t1; t += RPP) {
    float x[8], y[8];
    load8<T>(k + (int64_t)t * p.ksn, x);
    load8<T>(q + (int64_t)t * p.qsn, y);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] += x[e];
      s = fmaf(y[e], y[e], s);
    }
    qm = fmaxf(qm, row_sum(s, TPR));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sh[r][col * 8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
    for (int i = 0; i < RPP; ++i) s += sh[i][threadIdx.x];
    p.ws_part[((int64_t)bh * NC + c) * D + threadIdx.x] = s;
  }
  const float m = block_max(qm, red);
  if (threadIdx.x == 0) p.ws_qmax[(int64_t)bh * NC + c] = m;
}

// Per (frame, head): the frame's key sum from its chunks' partial sums, in
// chunk order.
template <int D>
__global__ __launch_bounds__(D) void bounds_frames(BoundsParams p) {
  const int f = blockIdx.x, bh = blockIdx.y;
  const int NC = p.F * p.chunks_per_frame;
  const int j = threadIdx.x;
  const float *part = p.ws_part + ((int64_t)bh * NC + (int64_t)f * p.chunks_per_frame) * D + j;
  p.ws_frame[((int64_t)bh * p.F + f) * D + j] = ordered_sum(part, p.chunks_per_frame, D);
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bounds_pass2(BoundsParams p) {
  constexpr int TPR = D / 8;
  constexpr int RPP = kThreads / TPR;
  __shared__ float red[kThreads];
  __shared__ float mu_sh[D];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.H, h = bh % p.H;
  const int NC = p.F * p.chunks_per_frame;
  // key mean of the head: frame sums added in frame order, divided by N
  // (every workgroup of the head computes the same bits; chunk 0 stores it)
  if (threadIdx.x < D) {
    const float *S = p.ws_frame + (int64_t)bh * p.F * D + threadIdx.x;
    const float mu = ordered_sum(S, p.F, D) / (float)p.N;
    mu_sh[threadIdx.x] = mu;
    if (c == 0) p.key_mean[(int64_t)bh * D + threadIdx.x] = mu;
  }
  __syncthreads();
  const int col = threadIdx.x % TPR, r = threadIdx.x / TPR;
  const T *k = static_cast<const T *>(p.k) + b * p.ksb + h * p.ksh + col * 8;
  float mu[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = mu_sh[col * 8 + e];
  int t0, t1;
  chunk_range(p, c, &t0, &t1);
  float km = 0.f;
  for (int t = t0 + r; t < t1; t += RPP) {
    float x[8];
    load8<T>(k + (int64_t)t * p.ksn, x);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float dlt = x[e] - mu[e];
      s = fmaf(dlt, dlt, s);
    }
    km = fmaxf(km, row_sum(s, TPR));
  }
  const float m = block_max(km, red);
  if (threadIdx.x == 0) p.ws_kmax[(int64_t)bh * NC + c] = m;
}

constexpr int kFinalLdsFloats = 12288;   // frame sums staged in LDS up to this size (48 KB)

template <int D>
__global__ __launch_bounds__(kThreads) void bounds_final(BoundsParams p) {
  constexpr int PER_LANE = D / 64;
  __shared__ float red[kThreads];
  __shared__ float S_sh[kFinalLdsFloats];
  const int bh = blockIdx.x;
  const int NC = p.F * p.chunks_per_frame;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float *Sg = p.ws_frame + (int64_t)bh * p.F * D;
  const bool staged = p.F * D <= kFinalLdsFloats;
  if (staged)
    for (int i = threadIdx.x; i < p.F * D; i += kThreads) S_sh[i] = Sg[i];
  float km = 0.f, qm = 0.f;
  for (int c = threadIdx.x; c < NC; c += kThreads) {
    km = fmaxf(km, p.ws_kmax[(int64_t)bh * NC + c]);
    qm = fmaxf(qm, p.ws_qmax[(int64_t)bh * NC + c]);
  }
  km = block_max(km, red);   // (its barriers also publish S_sh)
  qm = block_max(qm, red);
  float mu[PER_LANE];
#pragma unroll
  for (int e = 0; e < PER_LANE; ++e) mu[e] = p.key_mean[(int64_t)bh * D + lane + 64 * e];
  const float *S = staged ? S_sh : Sg;
  // c_max: the largest distance between the mean of the keys a query frame
  // sees (its window plus the reference frame) and the head's key mean.
  // One wave per frame; the squared distance is summed over the wave.
  float cm = 0.f;
  for (int f = wave; f < p.F; f += kThreads / 64) {
    const int lo = max(0, f - p.wr), hi = min(p.F - 1, f + p.wa);
    const bool extra = p.ref >= 0 && (p.ref < lo || p.ref > hi);
    const float cnt = (float)(hi - lo + 1 + (extra ? 1 : 0)) * (float)p.T;
    float dd = 0.f;
#pragma unroll
    for (int e = 0; e < PER_LANE; ++e) {
      const int j = lane + 64 * e;
      float w = 0.f;
      if (extra && p.ref < lo) w += S[(int64_t)p.ref * D + j];
      w += ordered_sum(S + (int64_t)lo * D + j, hi - lo + 1, D);
      if (extra && p.ref > hi) w += S[(int64_t)p.ref * D + j];
      const float dlt = w / cnt - mu[e];
      dd = fmaf(dlt, dlt, dd);
    }
    for (int o = 32; o > 0; o >>= 1) dd += __shfl_xor(dd, o, 64);
    cm = fmaxf(cm, dd);
  }
  cm = block_max(cm, red);
  if (threadIdx.x == 0) {
    const float qn = sqrtf(qm);
    const float kn = sqrtf(km);
    const float cn = sqrtf(cm);
    fsattn_head_bound r;
    r.q_norm_max = qn;
    r.k_norm_max = kn;
    r.c_max = cn;
    r.bound = p.scale * qn * kn;
    r.gap_est = p.scale * qn * (kn + cn);
    r.eligible = r.gap_est <= p.threshold ? 1 : 0;
    r.pad[0] = r.pad[1] = 0;
    p.rec[bh] = r;
  }
}

template <typename T, int D>
hipError_t launch_all(const BoundsParams &p, hipStream_t st) {
  const int BH = p.B * p.H;
  const int NC = p.F * p.chunks_per_frame;
  hipLaunchKernelGGL((bounds_pass1<T, D>), dim3(NC, BH), dim3(kThreads), 0, st, p);
  hipLaunchKernelGGL((bounds_frames<D>), dim3(p.F, BH), dim3(D), 0, st, p);
  hipLaunchKernelGGL((bounds_pass2<T, D>), dim3(NC, BH), dim3(kThreads), 0, st, p);
  hipLaunchKernelGGL((bounds_final<D>), dim3(BH), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_head_bounds(const BoundsParams &p, int dtype, hipStream_t st) {
  if (dtype == FSATTN_BF16) {
    if (p.D == 128) return launch_all<__hip_bfloat16, 128>(p, st);
    return launch_all<__hip_bfloat16, 64>(p, st);
  }
  if (p.D == 128) return launch_all<float, 128>(p, st);
  return launch_all<float, 64>(p, st);
}

}  // namespace fsattn
