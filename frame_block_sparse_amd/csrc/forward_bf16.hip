// bf16 forward on MFMA: frame-block-sparse attention for gfx950.
//
// "HeyGen x Google Cloud: Bringing Avatar IV to TPUs":
//  * "Deleting the Mask": blocks that divide the frame span are full or
//    empty, so the inner loop is a dense attention loop over the live key
//    ranges of the plan (window and reference frame in one pass), with no
//    mask predicate, no padding and no second pass.
//  * "Unchaining the Softmax", Fig. 4: on eligible heads every row starts
//    with a precomputed shift derived from the small per-head record
//    (Cauchy-Schwarz bound of the mean-centred logits plus scale*q_i.mu), so
//    the inner loop has no running max and no rescaling; other heads take
//    the online path (running max, rescale) inside the same kernel.
//  * "Proving the Pixels Didn't Change": the final product PV runs in bf16 on
//    the matrix unit (P rounded to bf16), accumulating in fp32.
//
// Work decomposition. A workgroup of W waves owns up to R = W * 16 * M16
// query rows of one frame of one (batch, head); all its rows share the
// frame's key list, so each K/V step is staged once in LDS and reused by
// every wave. A wave owns 16 * M16 rows, which must divide the frame span;
// when W wave tiles do not divide it, the frame's last workgroup has idle
// waves (they still help stage K/V). Per 32-key chunk of a step:
//   S^T = K Q^T      v_mfma_f32_16x16x32_bf16, A = K rows from LDS, B = Q
//                    held in registers; lane (g = lane/16, n = lane%16)
//                    ends with S[q = n][keys 4g..4g+3] of each 16-key tile
//   softmax          fp32 exp2 on those registers; the row statistics of
//                    query n live in the four lanes n, n+16, n+32, n+48
//   O^T += V^T P^T   the same MFMA with A = V^T read by ds_read_b64_tr_b16
//                    (4 keys x 1 column per lane, hardware transpose) and
//                    B = P^T, which is exactly the lane's own S registers
//                    converted to bf16; a 16-key tail uses the 16x16x16 MFMA
// so P never leaves registers and O's rows sit in the same lanes as S's.
//
// Staging. K/V steps go global -> LDS with global_load_lds_dwordx4 (no
// registers in between): each wave instruction writes 1 KB of consecutive
// LDS, so rows are unpadded and bank conflicts (64 banks of 4 bytes) are
// removed by XOR swizzles instead: K rows swizzle 16-byte chunks so that
// the 16 rows one operand read touches fall on 16 different bank groups;
// V rows swizzle 32-byte segments (the unit of a transposed read) so that
// the 8 rows two lane groups read together fall on 8 different ones.
// NBUF buffers form a ring:
// while step s is computed, steps s+1 .. s+NBUF-1 are in flight. Every step
// issues the same number of copies per wave (a short step re-reads its last
// valid row), so each wave waits only for its own copies of step s with a
// constant vmcnt, and one barrier per step publishes them to all waves.
//
// Order. Workgroups are issued heavy frames first (frames seeing the most
// key frames), and the tiles, in chunks of consecutive tiles of one (frame,
// head) group, are dealt round-robin to the 8 XCDs, so that tiles that
// stream the same K/V run on one XCD and share its L2; the chunk size
// balances the XCDs' work (fsattn_schedule.cpp).
#include <hip/hip_runtime.h>

#include <mutex>

#include "forward_common.h"

namespace fsattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned u4 __attribute__((ext_vector_type(4)));
typedef unsigned u2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) short4v lds_short4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_uchar;
typedef __attribute__((address_space(1))) void glb_void;

__device__ inline f4 mfma32(bf16x8 a, bf16x8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f4 mfma16(bf16x4 a, bf16x4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// Transposed LDS read: the 16 lanes of a group address a 4 x 16 block
// (row j/4, columns 4*(j%4)..+3 for lane j); lane i receives column i of
// the four rows.
__device__ inline bf16x4 lds_read_tr(unsigned addr) {
  const short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4 *)(uintptr_t)addr);
  return __builtin_bit_cast(bf16x4, r);
}
// 16-byte LDS read at an LDS byte address.
__device__ inline bf16x8 lds_read16(unsigned addr) { return *(const lds_bf16x8 *)(uintptr_t)addr; }

// Reductions over the four lanes n, n+16, n+32, n+48 that hold one row's
// statistics: v_permlane16_swap / v_permlane32_swap leave every lane with
// its own value and the one of lane l ^ 16 (l ^ 32), in either order, so
// the max or sum of the two is the pair's (VALU ops, no LDS round trip).
__device__ inline float pair_max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float pair_sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float row_max4(float v) { return pair_max32(pair_max16(v)); }
__device__ inline float row_sum4(float v) { return pair_sum32(pair_sum16(v)); }

// acc + x.lo + x.hi for a packed bf16 pair (v_dot2c_f32_bf16 with (1, 1)).
__device__ inline float add_bf16_pair(float acc, unsigned x) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, acc, false);
}

// One wave-wide global -> LDS copy of 16 bytes per lane
// (global_load_lds_dwordx4): lane l's bytes land at LDS address lds + 16*l.
// Issued from inline assembly so that the compiler's wait insertion, which
// cannot tell the two staging buffers apart, does not stall every LDS read
// behind the in-flight prefetch; completion is awaited explicitly
// (wait_vmem() before the step barrier). M0 carries the LDS base.
// The address is a wave-uniform 64-bit base (SGPR pair) plus a 32-bit
// per-lane byte offset.
__device__ inline uint64_t uniform_u64(uint64_t a) {
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ inline uint64_t uniform_ptr(const void *p) { return uniform_u64(reinterpret_cast<uint64_t>(p)); }
// (the scalar operands pass through readfirstlane, which only states what
// they already are: wave-uniform; M0 is declared clobbered, so the compiler
// keeps no value of its own in it across the copy)
__device__ inline void dma16(uint64_t base, unsigned off, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(uniform_u64(base)),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// s_waitcnt vmcnt(0) through the builtin, which the compiler's own wait
// tracking sees (it does not parse inline assembly): after it, no vector
// memory load is considered outstanding, so no wait for an earlier load is
// sunk into the step loop, where it would also stall on the prefetch.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// s_waitcnt vmcnt(N) (other counters unconstrained), N < 64.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup index -> (frame, batch*head, tile within the frame): tile t
// of XCD x's list (dealt_tile), whose issue-order index g numbers the
// tiles of (frame, head) group g / TPF, heaviest frames first. Returns false
// for a workgroup past the end of its XCD's list.
__device__ inline bool map_block(const FwdParams &p, int bid, int &f, int &bh, int &tile) {
  const int BH = p.B * p.H;
  const int TPF = p.tiles_per_frame;
  const int64_t G = (int64_t)p.F * BH * TPF;
  const int x = bid % kXcds, t = bid / kXcds;
  if (t >= xcd_tile_count(G, p.deal_chunk, x)) return false;
  const int64_t g = dealt_tile(G, p.deal_chunk, x, t);
  const int gi = (int)(g / TPF);
  tile = (int)(g % TPF);
  const int fr = gi / BH;
  bh = gi % BH;
  f = p.ordered ? p.frame_order[fr] : fr;
  return true;
}

// Waves per SIMD the register budget is held to: 3 for 32-row waves, 2 for
// 48-row waves, 1 above.
constexpr int fwd_min_waves(int m16) { return m16 <= 2 ? 3 : (m16 == 3 ? 2 : 1); }

// Online path: how far (log2 units) a row's maximum may pass its running
// shift before the wave rescales.
constexpr float kLazyRescaleLog2 = 8.f;

// PRIOR instantiates the prior-art comparator instead of the method: one
// pass (window or reference frame) over 128-row query tiles of the padded
// sequence, keys in 128-key tiles with a per-element frame predicate on the
// tiles that are only partly live, online softmax, normalised fp32 rows and
// log-sum-exps out (the merge of the two passes is a separate kernel).
template <int M16, int W, int NK16, int NBUF, int D, bool PRIOR = false>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(fwd_min_waves(M16))))
void fwd_bf16_kernel(FwdParams p) {
  constexpr int NK = NK16 * 16;
  constexpr int KD = D / 32;          // 32-wide slices of d for QK^T
  constexpr int DT = D / 16;          // 16-wide output column tiles for PV
  constexpr int ROWB = 2 * D;         // bytes per K/V row in LDS
  constexpr int TILEB = NK * ROWB;    // bytes of one K (or V) tile
  constexpr int RPI = 1024 / ROWB;    // rows written by one wave-wide 16-byte load
  constexpr int NI = NK / RPI;        // such loads per tile
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  // Register prefetch of K and V fragments (below) fits the register budget
  // of 32-key steps with at least 4 waves; the other shapes spill with it.
  constexpr bool PF = NK16 == 2 && W >= 4;
  // swizzles: K chunk c of row r lives at chunk c ^ ksw(r); V 32-byte
  // segment s of row r lives at segment s ^ vsw(r). Rows are 256 bytes for
  // d = 128 (one full bank row), 128 bytes for d = 64 (two rows per bank row).
  auto ksw = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto vsw = [](int r) { return D == 128 ? (r & 7) : ((r >> 1) & 3); };
  static_assert(NBUF >= 2, "ring of at least two buffers");

  extern __shared__ __align__(16) unsigned char smem[];
  // NBUF x [K tile, V tile], then the runs
  int2 *runs = reinterpret_cast<int2 *>(smem + 2 * NBUF * TILEB);
  int *nruns_sm = reinterpret_cast<int *>(runs + kMaxRuns);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < W);
  const int g = lane >> 4, n16 = lane & 15;
  int f, bh, ti;
  if constexpr (PRIOR) {
    static_assert(!PRIOR || (NK16 == 2 && W * 16 * M16 == 128), "comparator: 128-row tiles, 32-key steps");
    f = 0;
    ti = blockIdx.x % p.tiles128;
    bh = blockIdx.x / p.tiles128;
  } else {
    if (!map_block(p, blockIdx.x, f, bh, ti)) return;
  }
  const int b = bh / p.H, h = bh % p.H;
  const int row0 = PRIOR ? ti * 128 : f * p.T + ti * p.rows_per_wg;
  const int fend = PRIOR ? p.N : (f + 1) * p.T;   // the frame's end row (comparator: the sequence's)
  // A wave whose 16 * M16 rows run past the frame's end (when they do not
  // divide the frame span) computes its rows past the end on the frame's
  // last query row and does not store them.
  const bool active = row0 + wave * 16 * M16 < fend;   // wave-uniform

  const __bf16 *qb = static_cast<const __bf16 *>(p.q) + b * p.qsb + h * p.qsh;
  // K and V bases of this (batch, head) as wave-uniform byte addresses: the
  // copies' addresses are computed on the scalar unit
  const uint64_t kb = uniform_ptr(static_cast<const __bf16 *>(p.k) + b * p.ksb + h * p.ksh);
  const uint64_t vb = uniform_ptr(static_cast<const __bf16 *>(p.v) + b * p.vsb + h * p.vsh);
  const int wrow0 = row0 + wave * 16 * M16;

  // Prologue loads, issued together so that their latencies overlap (and
  // overlap the plan reads of wave 0 and the first K/V copies below): the Q
  // fragments (B operand of S^T = K Q^T: row n16 of each 16-row group,
  // d = 32*kd + 8*g .. +7) and, unless every head runs online, the head's
  // record and this lane's slices of its mean key.
  // An idle wave reads its workgroup's first rows instead (always in range)
  // and never stores.
  const int qrow0 = active ? wrow0 : row0;
  bf16x8 qf[M16][KD];
#pragma unroll
  for (int m = 0; m < M16; ++m)
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
      qf[m][kd] = *reinterpret_cast<const bf16x8 *>(qb + (int64_t)min(qrow0 + 16 * m + n16, fend - 1) * p.qsn +
                                                     32 * kd + 8 * g);
  const int mode = p.flags & 3;
  const bool may_fix = !PRIOR && mode != FSATTN_MODE_FORCE_ONLINE;   // key_mean and rec are given
  int eligible = 0;
  float bound = 0.f, kmax = 0.f;
  float4 muv[KD][2];
  if (may_fix) {
    eligible = p.rec[bh].eligible;
    bound = p.rec[bh].bound;
    kmax = p.rec[bh].k_norm_max;
    const float4 *mu4 = reinterpret_cast<const float4 *>(p.key_mean + (int64_t)bh * D + 8 * g);
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      muv[kd][0] = mu4[8 * kd];
      muv[kd][1] = mu4[8 * kd + 1];
    }
  }
  if (!PRIOR && wave == 0) build_runs(p.row_ptr, p.col_idx, p.nnz, row0 / p.bq, p.bk, p.N, runs, nruns_sm);

  // Row sums: the online path adds the probabilities with v_dot2c (it
  // rescales the sum with one multiply); the fixed path sums them on the
  // matrix unit, as O's column tile of an all-ones V, which every lane of a
  // row then holds whole (4 copies).
  float lsum[M16];
  f4 lsum4[M16];
  f4 oacc[M16][DT];
#pragma unroll
  for (int m = 0; m < M16; ++m) {
    lsum[m] = 0.f;
    lsum4[m] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[m][dt] = f4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = p.scale_log2;

  __syncthreads();
  // The frame mask gives every query frame at most two runs of live keys
  // (the window, and the reference frame when it is not adjacent to it);
  // the host rejects masks with more. Their bounds live in scalar registers.
  int r0s, r0e, r1s, r1e;
  // comparator: the frames the tile's rows span, and its one key run
  [[maybe_unused]] int pfa = 0, pfb = 0;
  if constexpr (PRIOR) {
    const int last = min(row0 + 128, p.N) - 1;
    pfa = row0 / p.T;
    pfb = last / p.T;
    int ks, ke;
    if (p.prior_pass == 0) {
      ks = max(0, pfa - p.wb) * p.T;
      ke = (min(p.F - 1, pfb + p.wa) + 1) * p.T;
    } else {
      ks = p.ref * p.T;
      ke = (p.ref + 1) * p.T;
    }
    // whole 128-key tiles of the padded sequence
    r0s = ks & ~127;
    r0e = min((ke + 127) & ~127, p.tiles128 * 128);
    r1s = r1e = 0;
  } else {
    const int nr = min(*nruns_sm, 2);
    r0s = nr > 0 ? __builtin_amdgcn_readfirstlane(runs[0].x) : 0;
    r0e = nr > 0 ? __builtin_amdgcn_readfirstlane(runs[0].y) : 0;
    r1s = nr > 1 ? __builtin_amdgcn_readfirstlane(runs[1].x) : 0;
    r1e = nr > 1 ? __builtin_amdgcn_readfirstlane(runs[1].y) : 0;
  }
  // Steps: first the F0 full NK-key steps of run 0 and the F1 of run 1,
  // then the short remainder of each run that has one (16 * k keys, k < NK
  // / 16): the order of the keys does not change the result, and the loop
  // over full steps then has no length test.
  const int len0 = r0e - r0s, len1 = r1e - r1s;
  const int F0 = len0 / NK, F1 = len1 / NK;
  const int nfull = F0 + F1;
  const int t0 = len0 - NK * F0, t1 = len1 - NK * F1;   // remainders
  const int nsteps = nfull + (t0 > 0) + (t1 > 0);
  // remainder step nfull + e: its run's first remainder row, end and length
  const int tpos0 = t0 > 0 ? r0s + NK * F0 : r1s + NK * F1, tend0 = t0 > 0 ? r0e : r1e;
  const int tlen0 = t0 > 0 ? t0 : t1;
  const int tpos1 = r1s + NK * F1, tend1 = r1e, tlen1 = t1;

  // Global -> LDS copies. A tile of NK rows is NI wave-wide copies of RPI
  // rows (copy c holds rows RPI*c ..). Lane l writes physical chunk l % CPR
  // of row RPI*c + l / CPR, which holds the logical chunk given by the
  // tile's swizzle. Both swizzles have period 16 rows, so copies whose rows
  // differ by a multiple of 16 read the same chunk of their rows: they form
  // one of G = 16 / RPI groups per tensor (copies p, p + G, ...), and a
  // lane's source offset within a full step is one value per group. The 2G
  // groups (K, then V) are dealt to the waves round-robin: wave w owns groups
  // w, w + W, ... (with more waves than groups some waves copy nothing).
  constexpr int G = 16 / RPI;             // groups per tensor
  constexpr int CPG = NI / G;             // copies per group per tile
  constexpr int GPW = (2 * G + W - 1) / W;   // group slots per wave
  static_assert(NI % G == 0, "a tile holds whole groups");
  // every wave owns the same number of groups (then a wave knows how many
  // of its copies are in flight per step)
  constexpr bool EVEN = (2 * G) % W == 0;
  constexpr int LPW = EVEN ? 2 * G / W * CPG : 0;   // copies per wave per step
  const int lrow = lane / CPR, lchunk = lane % CPR;
  // Byte offsets within a step are 32-bit (the host guarantees that 64 rows
  // of either tensor span less than 2^31 bytes).
  const unsigned kstride2 = (unsigned)(2 * p.ksn), vstride2 = (unsigned)(2 * p.vsn);
  const unsigned lds_base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_uchar *)smem);
  // this lane's source offset for copy c of K (or V) when the step has kl
  // rows (rows past kl re-read row kl - 1)
  auto src_off = [&](bool isv, int c, int kl) -> unsigned {
    const int r = RPI * c + lrow;
    const unsigned rs = (unsigned)min(r, kl - 1);
    if (!isv) return rs * kstride2 + 16u * (lchunk ^ ksw(r));
    return rs * vstride2 + 16u * ((((lchunk >> 1) ^ vsw(r)) << 1) | (lchunk & 1));
  };
  // the wave's groups and each one's lane offset in a full step
  unsigned goff[GPW];
#pragma unroll
  for (int sl = 0; sl < GPW; ++sl) {
    const int gi = wave + sl * W;
    goff[sl] = gi < 2 * G ? src_off(gi >= G, gi % G, NK) : 0u;
  }
  // The copy side walks the steps in order with the byte addresses of its
  // next step's first K and V rows, advanced by one step's stride and set
  // to run 1's first row when it gets there.
  const uint64_t kstep = 2 * (uint64_t)p.ksn, vstep = 2 * (uint64_t)p.vsn;   // bytes per row
  const uint64_t k1 = kb + (uint64_t)r1s * kstep, v1 = vb + (uint64_t)r1s * vstep;
  int lj = 0;
  uint64_t lkr = kb + (uint64_t)r0s * kstep, lvr = vb + (uint64_t)r0s * vstep;
  // A remainder step (kl < NK keys) reads the NK rows that end at its run's
  // end when the sequence has that many rows, so its copies take the same
  // per-lane offsets as a full step's and its live keys are the tile's last
  // kl rows; otherwise its rows past kl re-read row kl-1 and the live keys
  // are the first kl rows.
  const bool shift_short = p.N >= NK;
  // first row a remainder step copies, and its live rows' offset in the tile
  // (a multiple of 16 rows)
  const int trow0 = shift_short ? max(tend0 - NK, 0) : tpos0, toff0 = tpos0 - trow0;
  const int trow1 = shift_short ? max(tend1 - NK, 0) : tpos1, toff1 = tpos1 - trow1;
  auto issue_loads = [&](int buf, uint64_t kr, uint64_t vr, bool fast, int kl) {
    const unsigned tile = lds_base + 2 * buf * TILEB;
#pragma unroll
    for (int sl = 0; sl < GPW; ++sl) {
      const int gi = wave + sl * W;   // wave-uniform
      if (gi < 2 * G) {
        const bool isv = gi >= G;
        const int pg = gi % G;
        const uint64_t base = isv ? vr : kr, stp = isv ? vstep : kstep;
        const unsigned dst = tile + (isv ? TILEB : 0u);
#pragma unroll
        for (int i = 0; i < CPG; ++i) {
          const int c = pg + G * i;
          if (fast) dma16(base + (uint64_t)(16 * i) * stp, goff[sl], dst + (unsigned)(c * RPI * ROWB));
          else dma16(base, src_off(isv, c, kl), dst + (unsigned)(c * RPI * ROWB));
        }
      }
    }
  };
  // copies of step lj (< nsteps) into ring buffer buf
  auto issue_next = [&](int buf) {
    if constexpr (PRIOR) {
      // keys past the sequence's end are padding: those steps copy clamped
      // rows (never read past row N - 1) and the predicate masks them
      const int row = r0s + NK * lj;
      if (row + NK <= p.N) {
        issue_loads(buf, kb + (uint64_t)row * kstep, vb + (uint64_t)row * vstep, true, NK);
      } else {
        const int crow = min(row, p.N - 1);
        issue_loads(buf, kb + (uint64_t)crow * kstep, vb + (uint64_t)crow * vstep, false, p.N - crow);
      }
      ++lj;
      return;
    }
    if (lj < nfull) {
      if (lj == F0) {
        lkr = k1;
        lvr = v1;
      }
      issue_loads(buf, lkr, lvr, true, NK);
      lkr += NK * kstep;
      lvr += NK * vstep;
    } else {
      const bool e0 = lj == nfull;
      const int row = e0 ? trow0 : trow1;
      issue_loads(buf, kb + (uint64_t)row * kstep, vb + (uint64_t)row * vstep, shift_short, e0 ? tlen0 : tlen1);
    }
    ++lj;
  };

  // The ring's first NBUF-1 steps go out now, so the shift computation
  // below (which waits for the prologue loads) runs while they are in flight.
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j)
    if (lj < nsteps) issue_next(j);

  const bool fixed = !PRIOR && (mode == FSATTN_MODE_FORCE_FIXED || (mode == FSATTN_MODE_AUTO && eligible != 0));
  float sh[M16];   // fixed: the row's shift; online: the running max (log2 units)
  if (fixed) {
    const bool per_row = (p.flags & FSATTN_SHIFT_PER_ROW) != 0;
#pragma unroll
    for (int m = 0; m < M16; ++m) {
      float dot = 0.f, nq = 0.f;
#pragma unroll
      for (int kd = 0; kd < KD; ++kd)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float x = (float)qf[m][kd][t];
          const float4 mv = muv[kd][t >> 2];
          const float mu = (t & 3) == 0 ? mv.x : (t & 3) == 1 ? mv.y : (t & 3) == 2 ? mv.z : mv.w;
          dot = fmaf(x, mu, dot);
          nq = fmaf(x, x, nq);
        }
      dot = row_sum4(dot);
      nq = row_sum4(nq);
      const float mrow = per_row ? p.scale * (sqrtf(nq) * kmax + dot) : bound + p.scale * dot;
      sh[m] = mrow * kLog2e;
    }
  } else {
#pragma unroll
    for (int m = 0; m < M16; ++m) sh[m] = -INFINITY;
  }
  // Every prologue load is complete after this (it is also step 0's wait
  // with a two-buffer ring), so the compiler has no load of its own left to
  // wait for inside the step loop, where the wait would also cover the
  // prefetch.
  wait_vmem();

  // Per-lane LDS addresses of the MFMA operand reads in a tile at offset 0
  // of the ring whose first row is a multiple of 16 (both swizzles have
  // period 16 in the row, so they depend on the lane only); a read adds the
  // tile's offset, which in the step loop is a constant of the instruction.
  // K: this lane's 16-byte chunk of row n16 for d slice kd (tile t adds 16
  // rows). V: the 4 x 16 transposed block of rows 4g + n16/4 (+16 for the
  // second tile), output tile dt.
  unsigned kofs[KD], vofs[DT];
#pragma unroll
  for (int kd = 0; kd < KD; ++kd) kofs[kd] = lds_base + n16 * ROWB + 16 * ((4 * kd + g) ^ ksw(n16));
  {
    const int vr = 4 * g + (n16 >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vofs[dt] = lds_base + vr * ROWB + 8 * (n16 & 3) + 32 * (dt ^ vsw(vr));
  }
  auto kread = [&](unsigned tile, int kd, int t) { return lds_read16(kofs[kd] + tile + 16 * t * ROWB); };
  auto vread = [&](unsigned tile, int dt, int t) { return lds_read_tr(vofs[dt] + tile + 16 * t * ROWB); };

  // Comparator: each row's frame (rows past the end take the last row's),
  // and whether the 128-key tile holding step key0 is live for every row of
  // the query tile (then no predicate is needed).
  [[maybe_unused]] int rowf[M16];
  if constexpr (PRIOR) {
#pragma unroll
    for (int m = 0; m < M16; ++m) rowf[m] = min(wrow0 + 16 * m + n16, p.N - 1) / p.T;
  }
  [[maybe_unused]] auto prior_full = [&](int key0) {
    const int kt0 = key0 & ~127;
    if (row0 + 128 > p.N || kt0 + 128 > p.N) return false;
    const int kfa = kt0 / p.T, kfb = (kt0 + 127) / p.T;
    if (p.prior_pass == 0) return kfa >= pfb - p.wb && kfb <= pfa + p.wa;
    return kfa == p.ref && kfb == p.ref && (p.ref < pfa - p.wb || p.ref > pfb + p.wa);
  };

  // One chunk of NS 16-key tiles (NS = 2, or 1 for a 16-key tail) whose K
  // rows start at LDS byte offset kt (a multiple of 16 rows into a K tile;
  // the V rows sit TILEB further).
  auto chunk = [&](auto fixed_tag, auto ns_tag, unsigned kt, [[maybe_unused]] int key0,
                   [[maybe_unused]] bool full) {
    constexpr bool FIXED = decltype(fixed_tag)::value;
    constexpr int NS = decltype(ns_tag)::value;
    const unsigned vt = kt + TILEB;
    f4 s[M16][NS];
#pragma unroll
    for (int m = 0; m < M16; ++m)
#pragma unroll
      for (int t = 0; t < NS; ++t) s[m][t] = f4{0.f, 0.f, 0.f, 0.f};
    // With prefetch the K fragments are double-buffered in registers: the
    // reads for slice kd+1 are in flight while the MFMAs of slice kd issue
    // (scheduling fences keep the compiler from sinking them next to their
    // use).
    constexpr int KB = PF && NS == 2 ? 2 : 1;
    [[maybe_unused]] bf16x8 ka[KB][NS];
    auto kload = [&](int kd, int slot) {
#pragma unroll
      for (int t = 0; t < NS; ++t) ka[slot][t] = kread(kt, kd, t);
    };
    if constexpr (KB == 2) {
      kload(0, 0);
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) {
        if (kd + 1 < KD) kload(kd + 1, (kd + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NS; ++t)
#pragma unroll
          for (int m = 0; m < M16; ++m) s[m][t] = mfma32(ka[kd & 1][t], qf[m][kd], s[m][t]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int kd = 0; kd < KD; ++kd)
#pragma unroll
        for (int t = 0; t < NS; ++t) {
          const bf16x8 a = kread(kt, kd, t);
#pragma unroll
          for (int m = 0; m < M16; ++m) s[m][t] = mfma32(a, qf[m][kd], s[m][t]);
        }
    }
    if constexpr (PRIOR) {
      // per-element predicate on a partly live key tile: the key's frame
      // against the row's window (pass 0), or the reference frame for rows
      // whose window does not hold it (pass 1); padding keys are dead
      if (!full) {
        const int kf0 = key0 / p.T, kb1 = (kf0 + 1) * p.T;
#pragma unroll
        for (int m = 0; m < M16; ++m)
#pragma unroll
          for (int t = 0; t < NS; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = key0 + 16 * t + 4 * g + i;
              const int kf = kf0 + (key >= kb1 ? 1 : 0);
              const bool live = key < p.N && (p.prior_pass == 0
                                                  ? kf >= rowf[m] - p.wb && kf <= rowf[m] + p.wa
                                                  : kf == p.ref && (p.ref < rowf[m] - p.wb || p.ref > rowf[m] + p.wa));
              // a read-modify-write (not a masked move): the score register
              // was just written by an MFMA, and only an instruction that
              // reads it is held back until that write has landed
              s[m][t][i] = fminf(s[m][t][i], live ? INFINITY : -INFINITY);
            }
      }
    }
    if constexpr (!FIXED) {
      // Online softmax: raise the running shift to the rows' maxima when
      // some row of the wave exceeds its shift by more than 2^8 (any shift
      // at or above a row's maximum gives the same softmax, and weights up
      // to 2^8 are exact enough in fp32 sums and bf16 P), then rescale.
      float mn[M16];
      bool raised = false;
#pragma unroll
      for (int m = 0; m < M16; ++m) {
        float mx = s[m][0][0];
#pragma unroll
        for (int t = 0; t < NS; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[m][t][i]);
        mx = row_max4(mx);
        mn[m] = fmaxf(sh[m], mx * c2);
        // lazy: the running shift only has to keep exp2(s - shift) <= 2^8,
        // so the wave rescales when some row's max passes its shift by more
        raised |= mn[m] > sh[m] + kLazyRescaleLog2;
      }
      if (__any(raised)) {
#pragma unroll
        for (int m = 0; m < M16; ++m) {
          // (a comparator row still without a live key has -inf on both
          // sides: factor 1, not exp2(NaN))
          const float alpha = (PRIOR && sh[m] == mn[m]) ? 1.f : __builtin_amdgcn_exp2f(sh[m] - mn[m]);
          sh[m] = mn[m];
          lsum[m] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) oacc[m][dt] *= alpha;
        }
      }
    }
    // With prefetch the first VF-1 V fragments are requested before the
    // exponentials so that their latency hides behind them; each PV step
    // then requests fragment dt+VF-1.
    constexpr int VF = 3;
    constexpr bool VPF = PF && NS == 2;
    bf16x4 va[VF][2];
    if constexpr (VPF) {
#pragma unroll
      for (int j = 0; j < VF - 1; ++j) {
        va[j][0] = vread(vt, j, 0);
        va[j][1] = vread(vt, j, 1);
      }
    }
    bf16x8 pk[M16];
    bf16x4 pt[M16];
#pragma unroll
    for (int m = 0; m < M16; ++m) {
      // (a comparator row that has seen no live key yet keeps a max of -inf)
      const float nsh = (PRIOR && sh[m] == -INFINITY) ? 0.f : -sh[m];
#pragma unroll
      for (int t = 0; t < NS; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[m][t][i] = __builtin_amdgcn_exp2f(fmaf(s[m][t][i], c2, nsh));
      // the row sum adds the probabilities PV multiplies (bf16)
      if constexpr (NS == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pk[m][i] = (__bf16)s[m][0][i];
          pk[m][4 + i] = (__bf16)s[m][1][i];
        }
        if constexpr (FIXED) {
          const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                               (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
          lsum4[m] = mfma32(ones, pk[m], lsum4[m]);
        } else {
          const u4 w = __builtin_bit_cast(u4, pk[m]);
#pragma unroll
          for (int j = 0; j < 4; ++j) lsum[m] = add_bf16_pair(lsum[m], w[j]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) pt[m][i] = (__bf16)s[m][0][i];
        if constexpr (FIXED) {
          const bf16x4 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
          lsum4[m] = mfma16(ones, pt[m], lsum4[m]);
        } else {
          const u2 w = __builtin_bit_cast(u2, pt[m]);
#pragma unroll
          for (int j = 0; j < 2; ++j) lsum[m] = add_bf16_pair(lsum[m], w[j]);
        }
      }
    }
    if constexpr (VPF) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        if (dt + VF - 1 < DT) {
          va[(dt + VF - 1) % VF][0] = vread(vt, dt + VF - 1, 0);
          va[(dt + VF - 1) % VF][1] = vread(vt, dt + VF - 1, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 a = __builtin_shufflevector(va[dt % VF][0], va[dt % VF][1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int m = 0; m < M16; ++m) oacc[m][dt] = mfma32(a, pk[m], oacc[m][dt]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        if constexpr (NS == 2) {
          const bf16x8 a = __builtin_shufflevector(vread(vt, dt, 0), vread(vt, dt, 1), 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int m = 0; m < M16; ++m) oacc[m][dt] = mfma32(a, pk[m], oacc[m][dt]);
        } else {
          const bf16x4 a = vread(vt, dt, 0);
#pragma unroll
          for (int m = 0; m < M16; ++m) oacc[m][dt] = mfma16(a, pt[m], oacc[m][dt]);
        }
      }
    }
  };
  // The step loop, instantiated once per softmax path so that the two
  // paths never merge inside it (idle waves run it with copies only). It is
  // unrolled by the ring depth, so each step's buffer offset is a constant
  // that folds into the LDS instructions.
  auto main_loop = [&](auto fixed_tag, auto compute_tag) {
    constexpr bool COMPUTE = decltype(compute_tag)::value;
    // step i's copies in: wait, publish, refill the buffer step i-1 used
    auto step_in = [&](int i, int buf) {
      // my copies of step i are done once at most NBUF-2 later steps'
      // copies are outstanding
      if (EVEN && i + NBUF - 2 < nsteps) wait_vmcnt<(NBUF - 2) * LPW>();
      else wait_vmem();
      __syncthreads();   // every wave's copies of step i landed; step i-1's buffer is free
      if (lj < nsteps) issue_next((buf + NBUF - 1) % NBUF);
    };
    auto full_step = [&](int i, int buf) {
      step_in(i, buf);
      if constexpr (COMPUTE) {
#pragma unroll
        for (int c = 0; c < NK / 32; ++c) {
          if constexpr (PRIOR) {
            const int key0 = r0s + NK * i + 32 * c;
            chunk(fixed_tag, std::integral_constant<int, 2>{}, 2 * buf * TILEB + 32 * c * ROWB, key0,
                  prior_full(key0));
          } else {
            chunk(fixed_tag, std::integral_constant<int, 2>{}, 2 * buf * TILEB + 32 * c * ROWB, 0, true);
          }
        }
      }
    };
    int i = 0;
    // full steps, unrolled by the ring depth: each buffer offset is a
    // constant of the LDS instructions
    for (; i + NBUF <= nfull; i += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) full_step(i + u, u);
    }
    for (; i < nfull; ++i) full_step(i, i % NBUF);
    // remainder steps
    for (; i < nsteps; ++i) {
      const int buf = i % NBUF;
      step_in(i, buf);
      if constexpr (COMPUTE) {
        const bool e0 = i == nfull;
        const int kl = e0 ? tlen0 : tlen1;
        // the step's first live row in the tile
        const unsigned k0 = 2 * buf * TILEB + (unsigned)(e0 ? toff0 : toff1) * ROWB;
#pragma unroll
        for (int c = 0; c < NK / 32 - 1; ++c)
          if (c < (kl >> 5)) chunk(fixed_tag, std::integral_constant<int, 2>{}, k0 + 32 * c * ROWB, 0, true);
        if (kl & 16) chunk(fixed_tag, std::integral_constant<int, 1>{}, k0 + (kl & ~31) * ROWB, 0, true);
      }
    }
  };
  if (!active) {
    main_loop(std::true_type{}, std::false_type{});
    return;
  }
  if (fixed)
    main_loop(std::true_type{}, std::true_type{});
  else
    main_loop(std::false_type{}, std::true_type{});

  // Epilogue: the row sums (one cross-lane reduction on the online path),
  // normalise, store.
#pragma unroll
  for (int m = 0; m < M16; ++m) {
    float l;
    if (fixed) {
      l = lsum4[m][0];
    } else {
      l = lsum[m];
      l = row_sum4(l);
    }
    const int row = wrow0 + 16 * m + n16;
    if (row >= fend) continue;
    if constexpr (PRIOR) {
      // the pass's normalised rows and log-sum-exps (a row with no live key
      // in this pass: zeros and -inf)
      const int64_t rr = (int64_t)bh * p.N + row;
      float *orow = p.part_o + rr * D;
      const float inv0 = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f4 x = oacc[m][dt] * inv0;
        *reinterpret_cast<float4 *>(orow + 16 * dt + 4 * g) = make_float4(x[0], x[1], x[2], x[3]);
      }
      if (g == 0) p.part_lse[rr] = l > 0.f ? (sh[m] + log2f(l)) * kLn2 : -INFINITY;
      continue;
    }
    const float inv = 1.f / l;
    if (p.o_f32) {
      float *orow = static_cast<float *>(p.o) + b * p.osb + h * p.osh + (int64_t)row * p.osn;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f4 x = oacc[m][dt] * inv;
        *reinterpret_cast<float4 *>(orow + 16 * dt + 4 * g) = make_float4(x[0], x[1], x[2], x[3]);
      }
    } else {
      __bf16 *orow = static_cast<__bf16 *>(p.o) + b * p.osb + h * p.osh + (int64_t)row * p.osn;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f4 x = oacc[m][dt] * inv;
        bf16x4 y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = (__bf16)x[i];
        *reinterpret_cast<bf16x4 *>(orow + 16 * dt + 4 * g) = y;
      }
    }
    if (p.lse && g == 0) p.lse[(int64_t)bh * p.N + row] = (sh[m] + log2f(l)) * kLn2;
  }
}


template <int M16, int W, int NK16, int NBUF, int D, bool PRIOR = false>
hipError_t launch_one(const FwdParams &p, const FwdConfig &c, hipStream_t st) {
  auto kern = fwd_bf16_kernel<M16, W, NK16, NBUF, D, PRIOR>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [&] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  });
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL(kern, dim3((unsigned)c.grid), dim3(W * 64), c.lds_bytes, st, p);
  return hipGetLastError();
}

template <int M16, int W, int NK16, int NBUF, int D>
int occupancy_one(const FwdConfig &c) {
  auto kern = fwd_bf16_kernel<M16, W, NK16, NBUF, D>;
  static std::mutex mu;
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] > 0) return cache[dev];
  if (hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                          160 * 1024) != hipSuccess)
    return 0;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(kern), W * 64,
                                                   c.lds_bytes) != hipSuccess)
    return 0;
  cache[dev] = n;
  return n;
}

}  // namespace

// (rows per wave / 16, waves per workgroup) pairs built, in order of
// preference; the first whose wave tile (16 * M16 rows) divides the frame
// span wins.
static const int kShapes[][2] = {{2, 4}, {3, 4}, {1, 4}, {4, 4}, {2, 8}, {3, 2}, {4, 2}, {2, 2}};

// (keys per step / 16, ring buffers) built; the first is the default.
static const int kSteps[][2] = {{2, 2}, {2, 3}, {2, 4}, {4, 2}};

int fwd_bf16_lds_bytes(int nk16, int nbuf, int D) {
  return nbuf * 2 * (nk16 * 16) * (2 * D) + kMaxRuns * 8 + 16;
}

bool choose_fwd_config(const fsattn_shape *s, const fsattn_mask *m, uint32_t flags, FwdConfig *cfg) {
  const int T = m->tokens_per_frame;
  const int BH = s->batch * s->heads;
  if (s->dtype == FSATTN_F32) {
    const int R = f32_rows_per_wg(T);
    cfg->waves = 1;
    cfg->m16 = R / 16;
    cfg->nk16 = 1;
    cfg->nbuf = 1;
    cfg->lds_bytes = 2 * 16 * s->head_dim * 4 + kMaxRuns * 8 + 4;
    cfg->grid = (int64_t)m->num_frames * (T / R) * BH;
    return true;
  }
  const int wo = (flags >> 8) & 15, mo = (flags >> 12) & 15, so = (flags >> 16) & 15,
            bo = (flags >> 20) & 15;
  int nk16 = 0, nbuf = 0;
  for (const auto &st : kSteps)
    if ((!so || st[0] == so) && (!bo || st[1] == bo)) {
      nk16 = st[0];
      nbuf = st[1];
      break;
    }
  if (!nk16) return false;
  for (const auto &sh : kShapes) {
    const int m16 = sh[0], w = sh[1];
    if ((wo && w != wo) || (mo && m16 != mo)) continue;
    // the library's choice takes wave tiles that divide the frame span; an
    // explicit rows-per-wave override may leave a frame's last wave partly
    // past its end
    if (!mo && T % (16 * m16)) continue;
    // keep at least two workgroups per CU within the 160 KB of LDS
    if (2 * fwd_bf16_lds_bytes(nk16, nbuf, s->head_dim) > 160 * 1024) continue;
    const int wave_tiles = (T + 16 * m16 - 1) / (16 * m16);
    cfg->waves = w;
    cfg->m16 = m16;
    cfg->nk16 = nk16;
    cfg->nbuf = nbuf;
    // 48-row waves hold two workgroups per CU by their registers, so a
    // 4-buffer ring costs them no occupancy (+0.3-0.6 % on 3600-token frames)
    if (!so && !bo && m16 == 3 && 2 * fwd_bf16_lds_bytes(2, 4, s->head_dim) <= 160 * 1024) cfg->nbuf = 4;
    cfg->lds_bytes = fwd_bf16_lds_bytes(nk16, cfg->nbuf, s->head_dim);
    cfg->grid = (int64_t)m->num_frames * ((wave_tiles + w - 1) / w) * BH;
    return true;
  }
  return false;
}

template <int M, int W, int D>
hipError_t launch_steps(const FwdParams &p, const FwdConfig &c, hipStream_t st) {
  if (c.nk16 == 2 && c.nbuf == 2) return launch_one<M, W, 2, 2, D>(p, c, st);
  if (c.nk16 == 2 && c.nbuf == 3) return launch_one<M, W, 2, 3, D>(p, c, st);
  if (c.nk16 == 2 && c.nbuf == 4) return launch_one<M, W, 2, 4, D>(p, c, st);
  if (c.nk16 == 4 && c.nbuf == 2) return launch_one<M, W, 4, 2, D>(p, c, st);
  return hipErrorInvalidValue;
}

#define FSATTN_SHAPE_CASE(M, W)                                               \
  if (c.m16 == M && c.waves == W)                                             \
    return head_dim == 128 ? launch_steps<M, W, 128>(p, c, st) : launch_steps<M, W, 64>(p, c, st);

hipError_t launch_forward_bf16(const FwdParams &p, const FwdConfig &c, int head_dim, hipStream_t st) {
  FSATTN_SHAPE_CASE(2, 4)
  FSATTN_SHAPE_CASE(3, 4)
  FSATTN_SHAPE_CASE(1, 4)
  FSATTN_SHAPE_CASE(4, 4)
  FSATTN_SHAPE_CASE(2, 8)
  FSATTN_SHAPE_CASE(3, 2)
  FSATTN_SHAPE_CASE(4, 2)
  FSATTN_SHAPE_CASE(2, 2)
  return hipErrorInvalidValue;
}

template <int M, int W, int D>
static int occupancy_steps(const FwdConfig &c) {
  if (c.nk16 == 2 && c.nbuf == 2) return occupancy_one<M, W, 2, 2, D>(c);
  if (c.nk16 == 2 && c.nbuf == 3) return occupancy_one<M, W, 2, 3, D>(c);
  if (c.nk16 == 2 && c.nbuf == 4) return occupancy_one<M, W, 2, 4, D>(c);
  if (c.nk16 == 4 && c.nbuf == 2) return occupancy_one<M, W, 4, 2, D>(c);
  return 0;
}

#define FSATTN_OCC_CASE(M, W)                                                 \
  if (c.m16 == M && c.waves == W)                                             \
    return head_dim == 128 ? occupancy_steps<M, W, 128>(c) : occupancy_steps<M, W, 64>(c);

int fwd_bf16_occupancy(const FwdConfig &c, int head_dim) {
  FSATTN_OCC_CASE(2, 4)
  FSATTN_OCC_CASE(3, 4)
  FSATTN_OCC_CASE(1, 4)
  FSATTN_OCC_CASE(4, 4)
  FSATTN_OCC_CASE(2, 8)
  FSATTN_OCC_CASE(3, 2)
  FSATTN_OCC_CASE(4, 2)
  FSATTN_OCC_CASE(2, 2)
  return 0;
}

hipError_t launch_prior_pass_bf16(const FwdParams &p, int head_dim, hipStream_t st) {
  FwdConfig c;
  c.waves = 4;
  c.m16 = 2;
  c.nk16 = 2;
  c.nbuf = 2;
  c.lds_bytes = fwd_bf16_lds_bytes(2, 2, head_dim);
  c.grid = (int64_t)p.tiles128 * p.B * p.H;
  if (head_dim == 128) return launch_one<2, 4, 2, 2, 128, true>(p, c, st);
  if (head_dim == 64) return launch_one<2, 4, 2, 2, 64, true>(p, c, st);
  return hipErrorInvalidValue;
}

namespace {

// O = the two passes' rows weighted by their exp(lse) (the merge of the
// prior-art comparator). One thread per 4 output elements.
__global__ __launch_bounds__(256) void prior_merge_kernel(const float *o_w, const float *lse_w, const float *o_r,
                                                          const float *lse_r, int H, int N, int D4, void *o,
                                                          int o_f32, int64_t osb, int64_t osh, int64_t osn,
                                                          int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int64_t rr = idx / D4;
  const int c = (int)(idx % D4);
  const int bh = (int)(rr / N), n = (int)(rr % N);
  const int b = bh / H, h = bh % H;
  const float lw = lse_w[rr], lr = o_r ? lse_r[rr] : -INFINITY;
  const float mx = fmaxf(lw, lr);
  const float ww = lw == -INFINITY ? 0.f : expf(lw - mx), wr = lr == -INFINITY ? 0.f : expf(lr - mx);
  const float inv = 1.f / (ww + wr);
  const float4 a = reinterpret_cast<const float4 *>(o_w)[idx];
  float4 r4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (o_r) r4 = reinterpret_cast<const float4 *>(o_r)[idx];
  const float y[4] = {(a.x * ww + r4.x * wr) * inv, (a.y * ww + r4.y * wr) * inv, (a.z * ww + r4.z * wr) * inv,
                      (a.w * ww + r4.w * wr) * inv};
  const int64_t off = b * osb + h * osh + (int64_t)n * osn + 4 * c;
  if (o_f32) {
    *reinterpret_cast<float4 *>(static_cast<float *>(o) + off) = make_float4(y[0], y[1], y[2], y[3]);
  } else {
    bf16x4 z;
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = (__bf16)y[i];
    *reinterpret_cast<bf16x4 *>(static_cast<__bf16 *>(o) + off) = z;
  }
}

}  // namespace

hipError_t launch_prior_merge(const float *o_w, const float *lse_w, const float *o_r, const float *lse_r,
                              int B, int H, int N, int D, void *o, int o_f32, int64_t osb, int64_t osh,
                              int64_t osn, hipStream_t st) {
  const int64_t total = (int64_t)B * H * N * (D / 4);
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(prior_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, st, o_w, lse_w, o_r, lse_r, H, N,
                     D / 4, o, o_f32, osb, osh, osn, total);
  return hipGetLastError();
}

}  // namespace fsattn
