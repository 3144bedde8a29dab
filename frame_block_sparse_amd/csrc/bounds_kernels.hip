// Per-head bound record ("HeyGen x Google Cloud: Bringing Avatar IV to
// TPUs", section "Unchaining the Softmax"): key mean, query-norm maximum,
// mean-centred key-norm maximum, the Cauchy-Schwarz logit bound, the window
// term c_max of the bound audit for windowed masks, and eligibility.
//
// Four launches; the two passes stream Q and K (HBM-bound), the other two
// are small. fsattn_produce runs the same four with the input-producing
// chain ("Layout Is the ABI", Fig. 5) fused into pass 1, whose statistics
// then come from the values it has just written:
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

#include <mutex>

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

// Round to the nearest bf16, ties to even (NaN stays NaN), and that value as
// a float.
__device__ inline uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Store 8 values and return, in x, the values as stored.
template <typename T>
__device__ inline void store8(T *p, float *x);

template <>
__device__ inline void store8<float>(float *p, float *x) {
  *reinterpret_cast<float4 *>(p) = float4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<float4 *>(p + 4) = float4{x[4], x[5], x[6], x[7]};
}

template <>
__device__ inline void store8<__hip_bfloat16>(__hip_bfloat16 *p, float *x) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = bf16_bits(x[2 * i]), hi = bf16_bits(x[2 * i + 1]);
    w[i] = lo | (hi << 16);
    x[2 * i] = __uint_as_float(lo << 16);
    x[2 * i + 1] = __uint_as_float(hi << 16);
  }
  *reinterpret_cast<uint4 *>(p) = uint4{w[0], w[1], w[2], w[3]};
}

// Copy 8 elements unchanged.
template <typename T>
__device__ inline void copy8(const T *src, T *dst) {
  if constexpr (sizeof(T) == 4) {
    const float4 a = *reinterpret_cast<const float4 *>(src), b = *reinterpret_cast<const float4 *>(src + 4);
    *reinterpret_cast<float4 *>(dst) = a;
    *reinterpret_cast<float4 *>(dst + 4) = b;
  } else {
    *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
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

// sum_{i < n} x[i * stride], added in index order, with up to 32 loads in
// flight (the order of the additions is the plain sequential one; a frame
// of 8160 tokens has 32 chunk sums, which then cost one round trip).
__device__ inline float ordered_sum(const float *x, int n, int64_t stride) {
  float s = 0.f;
  int i = 0;
  for (; i + 32 <= n; i += 32) {
    float v[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = x[(int64_t)(i + e) * stride];
#pragma unroll
    for (int e = 0; e < 32; ++e) s += v[e];
  }
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

// RMS normalisation of one token row held by `width` consecutive lanes, 8
// elements each: x <- g * x / sqrt(mean(x^2) + eps).
__device__ inline void rms_norm8(float *x, const float *g, int width, float inv_d, float eps) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
  ss = row_sum(ss, width);
  const float r = 1.f / sqrtf(ss * inv_d + eps);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = g[e] * (x[e] * r);
}

// Rotary embedding of 4 dimension pairs (2i, 2i+1): each pair is rotated by
// the angle whose cosine and sine are cs[i] and sn[i].
__device__ inline void rope8(float *x, const float *cs, const float *sn) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = x[2 * i], b = x[2 * i + 1];
    x[2 * i] = a * cs[i] - b * sn[i];
    x[2 * i + 1] = a * sn[i] + b * cs[i];
  }
}

// One token row of the input-producing chain: read Q, K and V, normalise and
// rotate Q and K, write all three, and return Q and K as written (yq, yk).
template <typename T, int D>
__device__ inline void produce_row(const BoundsParams &p, const ProduceParams &x, int b, int h, int64_t t,
                                   int col, const float *gq, const float *gk, float *yq, float *yk) {
  constexpr int TPR = D / 8;
  const T *qi = static_cast<const T *>(x.qi) + b * x.qisb + h * x.qish + t * x.qisn + col * 8;
  const T *ki = static_cast<const T *>(x.ki) + b * x.kisb + h * x.kish + t * x.kisn + col * 8;
  const T *vi = static_cast<const T *>(x.vi) + b * x.visb + h * x.vish + t * x.visn + col * 8;
  load8<T>(qi, yq);
  load8<T>(ki, yk);
  copy8<T>(vi, static_cast<T *>(x.vo) + b * x.vosb + h * x.vosh + t * x.vosn + col * 8);
  if (x.gq) rms_norm8(yq, gq, TPR, 1.f / D, x.eps);
  if (x.gk) rms_norm8(yk, gk, TPR, 1.f / D, x.eps);
  if (x.rcos) {
    const float4 c4 = *reinterpret_cast<const float4 *>(x.rcos + t * (D / 2) + col * 4);
    const float4 s4 = *reinterpret_cast<const float4 *>(x.rsin + t * (D / 2) + col * 4);
    const float cs[4] = {c4.x, c4.y, c4.z, c4.w}, sn[4] = {s4.x, s4.y, s4.z, s4.w};
    rope8(yq, cs, sn);
    rope8(yk, cs, sn);
  }
  store8<T>(static_cast<T *>(x.qo) + b * p.qsb + h * p.qsh + t * p.qsn + col * 8, yq);
  store8<T>(static_cast<T *>(x.ko) + b * p.ksb + h * p.ksh + t * p.ksn + col * 8, yk);
}

// PRODUCE: the input-producing chain is fused in (fsattn_produce); the key
// sums and query norms are then those of the values written, in the same
// order, so they equal what pass 1 alone computes on the outputs.
template <typename T, int D, bool PRODUCE>
__global__ __launch_bounds__(kThreads) void bounds_pass1(BoundsParams p, ProduceParams xp) {
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
  [[maybe_unused]] float gq[8], gk[8];
  if constexpr (PRODUCE) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gq[e] = xp.gq ? xp.gq[h * D + col * 8 + e] : 1.f;
      gk[e] = xp.gk ? xp.gk[h * D + col * 8 + e] : 1.f;
    }
  }
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float qm = 0.f;
  for (int t = t0 + r; t < t1; t += U * RPP) {
    float x[U][8], y[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u * RPP < t1) {
        if constexpr (PRODUCE) {
          produce_row<T, D>(p, xp, b, h, t + u * RPP, col, gq, gk, y[u], x[u]);
        } else {
          load8<T>(k + (int64_t)(t + u * RPP) * p.ksn, x[u]);
          load8<T>(q + (int64_t)(t + u * RPP) * p.qsn, y[u]);
        }
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

constexpr int kHeadThreads = 1024;
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
// estimate and eligibility. A key mean that is not finite (a key that is
// not) leaves the fixed shift without meaning, and the maxima skip NaN, so
// such a head is marked not eligible: the online path then confines the
// non-finite values to the rows that attend to them.
__global__ __launch_bounds__(kThreads) void bounds_final(BoundsParams p) {
  __shared__ float red[kThreads / 64];
  const int bh = blockIdx.x;
  const int NC = p.F * p.chunks_per_frame;
  float km = 0.f;
  for (int c = threadIdx.x; c < NC; c += kThreads) km = fmaxf(km, p.ws_kmax[(int64_t)bh * NC + c]);
  float bad = 0.f;
  for (int j = threadIdx.x; j < p.D; j += kThreads) bad = isfinite(p.key_mean[(int64_t)bh * p.D + j]) ? bad : 1.f;
  km = block_max<kThreads>(km, red);
  bad = block_max<kThreads>(bad, red);
  if (threadIdx.x == 0) {
    fsattn_head_bound r = p.rec[bh];   // q_norm_max and c_max from the head pass
    const float qn = r.q_norm_max, cn = r.c_max;
    const float kn = sqrtf(km);
    r.k_norm_max = kn;
    r.bound = p.scale * qn * kn;
    r.gap_est = p.scale * qn * (kn + cn);
    r.eligible = r.gap_est <= p.threshold && bad == 0.f ? 1 : 0;
    r.pad[0] = r.pad[1] = 0;
    p.rec[bh] = r;
  }
}

template <typename T, int D, bool PRODUCE = false>
hipError_t launch_all(const BoundsParams &p, hipStream_t st, const ProduceParams &x = ProduceParams{}) {
  const int BH = p.B * p.H;
  const int NC = p.F * p.chunks_per_frame;
  hipLaunchKernelGGL((bounds_pass1<T, D, PRODUCE>), dim3(NC, BH), dim3(kThreads), 0, st, p, x);
  hipLaunchKernelGGL((bounds_head<D>), dim3(BH), dim3(kHeadThreads), 0, st, p);
  hipLaunchKernelGGL((bounds_pass2<T, D>), dim3(NC, BH), dim3(kThreads), 0, st, p);
  hipLaunchKernelGGL(bounds_final, dim3(BH), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

// Workspace of fsattn_head_bounds_noalloc: one array per device, held from
// the time the library's code object is loaded until the process ends. The
// bounds kernels overwrite every partial result they later read, so nothing
// in it has to start at zero. In host code its name only stands for the
// symbol: the device address comes from hipGetSymbolAddress, once per
// device (each device holds its own copy at its own address).
static __device__ __align__(256) unsigned char scratch[kBoundsScratchBytes];

hipError_t bounds_scratch(void **ptr) {
  static std::mutex mu;
  static void *addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_head_bounds(const BoundsParams &p, int dtype, hipStream_t st) {
  if (dtype == FSATTN_BF16) {
    if (p.D == 128) return launch_all<__hip_bfloat16, 128>(p, st);
    return launch_all<__hip_bfloat16, 64>(p, st);
  }
  if (p.D == 128) return launch_all<float, 128>(p, st);
  return launch_all<float, 64>(p, st);
}

hipError_t launch_produce(const BoundsParams &p, const ProduceParams &x, int dtype, hipStream_t st) {
  if (dtype == FSATTN_BF16) {
    if (p.D == 128) return launch_all<__hip_bfloat16, 128, true>(p, st, x);
    return launch_all<__hip_bfloat16, 64, true>(p, st, x);
  }
  if (p.D == 128) return launch_all<float, 128, true>(p, st, x);
  return launch_all<float, 64, true>(p, st, x);
}

}  // namespace fsattn
