// Per-head bound record ("HeyGen x Google Cloud: Bringing Avatar IV to
// TPUs", section "Unchaining the Softmax"): key mean, query-norm maximum,
// mean-centred key-norm maximum, the Cauchy-Schwarz logit bound, the window
// term c_max of the bound audit for windowed masks, and eligibility.
//
// Four launches; the two passes stream Q and K (HBM-bound), the other two
// are small:
//   pass1   per (token chunk, head): partial key sums, partial max |q|^2
//   head    per head: the frame key sums from their chunks, the key mean,
//           c_max from the frame sums, max |q|
//   pass2   per (token chunk, head): partial max |k - mu|^2
//   final   per head: max |k - mu|, bound, gap estimate, eligibility
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

// Maximum over the workgroup (NT threads): within each wave by lane
// exchange, then over the waves' results in LDS (sh holds NT/64 floats).
// Every thread returns the maximum.
template <int NT>
__device__ inline float block_max(float v, float *sh) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int wave = threadIdx.x >> 6;
  __syncthreads();   // sh may still be read by a previous call
  if ((threadIdx.x & 63) == 0) sh[wave] = v;
  __syncthreads();
  float r = sh[0];
  for (int w = 1; w < NT / 64; ++w) r = fmaxf(r, sh[w]);
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
  constexpr int U = 4;                  // passes whose loads are issued together
  __shared__ float sh[RPP][D + 1];
  __shared__ float red[kThreads / 64];
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
  for (int t = t0 + r; t < t1; t += U * RPP) {
    float x[U][8], y[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u * RPP < t1) {
        load8<T>(k + (int64_t)(t + u * RPP) * p.ksn, x[u]);
        load8<T>(q + (int64_t)(t + u * RPP) * p.qsn, y[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[u][e] = y[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[e] += x[u][e];
        s = fmaf(y[u][e], y[u][e], s);
      }
      qm = fmaxf(qm, row_sum(s, TPR));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sh[r][col * 8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
    for (int i = 0; i < RPP; ++i) s += sh[i][threadIdx.x];
    p.ws_part[((int64_t)bh * NC + c) * D + threadIdx.x] = s;
  }
  const float m = block_max<kThreads>(qm, red);
  if (threadIdx.x == 0) p.ws_qmax[(int64_t)bh * NC + c] = m;
}

constexpr int kHeadThreads = 512;
constexpr int kHeadLdsFloats = 12288;   // frame sums staged in LDS up to this size (48 KB)

// Per head: the frame key sums (each the sum of its chunks' partial sums in
// chunk order), the key mean (frame sums added in frame order, divided by
// N), c_max from the frame sums, and max |q| from the chunk maxima.
template <int D>
__global__ __launch_bounds__(kHeadThreads) void bounds_head(BoundsParams p) {
  constexpr int PER_LANE = D / 64;
  constexpr int NW = kHeadThreads / 64;
  __shared__ float red[NW];
  __shared__ float S_sh[kHeadLdsFloats];
  __shared__ float mu_sh[D];
  const int bh = blockIdx.x;
  const int NC = p.F * p.chunks_per_frame;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // frame sums, wave w taking frames w, w + NW, ...; kept in LDS when they
  // fit, else in the workspace
  const bool staged = p.F * D <= kHeadLdsFloats;
  float *S = staged ? S_sh : p.ws_frame + (int64_t)bh * p.F * D;
  for (int f = wave; f < p.F; f += NW) {
    const float *part = p.ws_part + ((int64_t)bh * NC + (int64_t)f * p.chunks_per_frame) * D;
#pragma unroll
    for (int e = 0; e < PER_LANE; ++e)
      S[(int64_t)f * D + lane + 64 * e] = ordered_sum(part + lane + 64 * e, p.chunks_per_frame, D);
  }
  if (!staged) __threadfence();
  __syncthreads();
  if (!staged) __threadfence();
  if (threadIdx.x < D) {
    const float mu = ordered_sum(S + threadIdx.x, p.F, D) / (float)p.N;
    mu_sh[threadIdx.x] = mu;
    p.key_mean[(int64_t)bh * D + threadIdx.x] = mu;
  }
  float qm = 0.f;
  for (int c = threadIdx.x; c < NC; c += kHeadThreads) qm = fmaxf(qm, p.ws_qmax[(int64_t)bh * NC + c]);
  qm = block_max<kHeadThreads>(qm, red);   // (its barriers also publish mu_sh)
  float mu[PER_LANE];
#pragma unroll
  for (int e = 0; e < PER_LANE; ++e) mu[e] = mu_sh[lane + 64 * e];
  // c_max: the largest distance between the mean of the keys a query frame
  // sees (its window plus the reference frames; every frame for the queries
  // of global reference frames) and the head's key mean.
  // One wave per frame; the squared distance is summed over the wave.
  float cm = 0.f;
  for (int f = wave; f < p.F; f += NW) {
    int iv[4];
    const int nint = live_intervals(p.live, f, iv);
    const int n0 = iv[1] - iv[0] + 1, n1 = nint == 2 ? iv[3] - iv[2] + 1 : 0;
    const float cnt = (float)(n0 + n1) * (float)p.T;
    float dd = 0.f;
#pragma unroll
    for (int e = 0; e < PER_LANE; ++e) {
      const int j = lane + 64 * e;
      float w = ordered_sum(S + (int64_t)iv[0] * D + j, n0, D);
      if (n1) w += ordered_sum(S + (int64_t)iv[2] * D + j, n1, D);
      const float dlt = w / cnt - mu[e];
      dd = fmaf(dlt, dlt, dd);
    }
    for (int o = 32; o > 0; o >>= 1) dd += __shfl_xor(dd, o, 64);
    cm = fmaxf(cm, dd);
  }
  cm = block_max<kHeadThreads>(cm, red);
  if (threadIdx.x == 0) {
    p.rec[bh].q_norm_max = sqrtf(qm);
    p.rec[bh].c_max = sqrtf(cm);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bounds_pass2(BoundsParams p) {
  constexpr int TPR = D / 8;
  constexpr int RPP = kThreads / TPR;
  constexpr int U = 4;
  __shared__ float red[kThreads / 64];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.H, h = bh % p.H;
  const int NC = p.F * p.chunks_per_frame;
  const int col = threadIdx.x % TPR, r = threadIdx.x / TPR;
  const T *k = static_cast<const T *>(p.k) + b * p.ksb + h * p.ksh + col * 8;
  float mu[8];   // the key mean from the head pass
#pragma unroll
  for (int e = 0; e < 8; ++e) mu[e] = p.key_mean[(int64_t)bh * D + col * 8 + e];
  int t0, t1;
  chunk_range(p, c, &t0, &t1);
  float km = 0.f;
  for (int t = t0 + r; t < t1; t += U * RPP) {
    float x[U][8];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ok[u] = t + u * RPP < t1;
      if (ok[u]) load8<T>(k + (int64_t)(t + u * RPP) * p.ksn, x[u]);
      else
#pragma unroll
        for (int e = 0; e < 8; ++e) x[u][e] = mu[e];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dlt = x[u][e] - mu[e];
        s = fmaf(dlt, dlt, s);
      }
      km = fmaxf(km, row_sum(s, TPR));
    }
  }
  const float m = block_max<kThreads>(km, red);
  if (threadIdx.x == 0) p.ws_kmax[(int64_t)bh * NC + c] = m;
}

// Per head: max |k - mu| from the chunk maxima, then the bound, the gap
// estimate and eligibility.
__global__ __launch_bounds__(kThreads) void bounds_final(BoundsParams p) {
  __shared__ float red[kThreads / 64];
  const int bh = blockIdx.x;
  const int NC = p.F * p.chunks_per_frame;
  float km = 0.f;
  for (int c = threadIdx.x; c < NC; c += kThreads) km = fmaxf(km, p.ws_kmax[(int64_t)bh * NC + c]);
  km = block_max<kThreads>(km, red);
  if (threadIdx.x == 0) {
    fsattn_head_bound r = p.rec[bh];   // q_norm_max and c_max from the head pass
    const float qn = r.q_norm_max, cn = r.c_max;
    const float kn = sqrtf(km);
    r.k_norm_max = kn;
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
  hipLaunchKernelGGL((bounds_head<D>), dim3(BH), dim3(kHeadThreads), 0, st, p);
  hipLaunchKernelGGL((bounds_pass2<T, D>), dim3(NC, BH), dim3(kThreads), 0, st, p);
  hipLaunchKernelGGL(bounds_final, dim3(BH), dim3(kThreads), 0, st, p);
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
