/*
 * fsattn - frame-structured block-sparse attention for AMD MI355X (gfx950).
 *
 * C ABI of the library libfsattn.so. Three calls make the hot path:
 *   fsattn_plan         live key blocks per query block (host, bit-exact)
 *                       (fsattn_plan_device: the same arrays written on the GPU)
 *   fsattn_head_bounds  key mean, norm maxima, logit bound, eligibility (GPU)
 *   fsattn_forward      attention over the live blocks, fixed-shift or
 *                       online softmax chosen per head (GPU)
 * and fsattn_produce, the chain that makes Q, K and V (normalisation and
 * rotary embedding) fused with fsattn_head_bounds (GPU).
 *
 * The method is the one described in "HeyGen x Google Cloud: Bringing
 * Avatar IV to TPUs" (Google Developers Blog). Section names below refer to
 * the headings of that post.
 *
 * Conventions shared by every call:
 *  - Ownership: the caller owns every buffer, host or device. The library
 *    never allocates device memory and never synchronises a stream. Its
 *    global state: caches of launch choices per device and geometry, the
 *    device address of fsattn_head_bounds_noalloc's workspace per device
 *    (both thread-safe), and that workspace itself, a fixed array in the
 *    library's code object on each device it runs on.
 *  - Errors: arguments are validated on the host before any launch. On any
 *    error nothing is launched and no output is written. A failed launch is
 *    reported as FSATTN_ERR_HIP. Device faults surface on the stream.
 *  - Streams: `hip_stream` is a hipStream_t passed as void*; NULL means the
 *    null stream. GPU calls are asynchronous on that stream.
 *  - Layout ("Layout Is the ABI": the producer's layout is consumed as is,
 *    no repack): every tensor is [B, H, N, d] with arbitrary element strides
 *    for B, H and N and unit stride along d. Data pointers and the N stride
 *    in bytes must be multiples of 16.
 *  - Tokens are frame-major: token t belongs to frame t / tokens_per_frame.
 */
#ifndef FSATTN_H
#define FSATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FSATTN_ABI_VERSION 3

typedef enum fsattn_status {
  FSATTN_OK = 0,
  FSATTN_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad stride, size mismatch */
  FSATTN_ERR_BLOCK_GEOMETRY = 2,   /* blocks not multiples of 16 dividing the frame span */
  FSATTN_ERR_UNSUPPORTED = 3,      /* head_dim / dtype combination not built */
  FSATTN_ERR_BUFFER_TOO_SMALL = 4, /* caller buffer shorter than required */
  FSATTN_ERR_HIP = 5               /* a HIP runtime call or launch failed */
} fsattn_status;

/* Element types. */
enum { FSATTN_F32 = 0, FSATTN_BF16 = 1 };

/*
 * The frame-structured mask and its block tiling ("Deleting the Mask",
 * Fig. 3). Query frame f sees the key frames of the window
 * [f - window_before, f + window_after] clamped to [0, num_frames - 1],
 * plus the reference frames: ref_count consecutive frames from ref_frame
 * (ref_frame -1: none; ref_count 0 or 1: the one frame ref_frame; the span
 * must end inside the sequence). block_q and block_k must
 * be positive multiples of 16 that divide tokens_per_frame, so that every
 * block is entirely live or entirely masked.
 *
 * ref_queries_global (0 or 1) widens the reference frames to global tokens
 * in both directions, the symmetric reading of a "global" frame: with 1,
 * the reference frames' own queries see every key frame, instead of only
 * their window. The section describes the reference frame only as keys
 * every frame attends to, so 0 (keys only) is the default reading. Without
 * a reference frame (ref_frame = -1) ref_queries_global and ref_count have
 * no effect. Other values (ref_queries_global not 0 or 1, a negative
 * ref_count, a span past the last frame) are geometry errors.
 */
typedef struct fsattn_mask {
  int32_t num_frames;
  int32_t tokens_per_frame;
  int32_t window_before;
  int32_t window_after;
  int32_t ref_frame;
  int32_t block_q;
  int32_t block_k;
  int32_t ref_queries_global;
  int32_t ref_count;
} fsattn_mask;

/* Problem shape. seq_len must equal num_frames * tokens_per_frame.
 * head_dim is 64 or 128. dtype is FSATTN_F32 or FSATTN_BF16 and applies to
 * Q, K and V alike. */
typedef struct fsattn_shape {
  int32_t batch;
  int32_t heads;
  int32_t seq_len;
  int32_t head_dim;
  int32_t dtype;
} fsattn_shape;

/* A strided [B, H, N, d] device tensor. Strides are in elements. */
typedef struct fsattn_tensor {
  void *data;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_n;
} fsattn_tensor;

/*
 * Per-(batch, head) record written by fsattn_head_bounds ("Unchaining the
 * Softmax": the small array of precomputed norms the kernel reads as each
 * row starts). All values use the softmax scale passed to the call.
 *   q_norm_max = max_i |q_i|
 *   k_norm_max = max_j |k_j - mu|            (mu = key mean of the head)
 *   c_max      = max_f |kbar_f - mu|         (kbar_f = mean of the keys
 *                                             live for query frame f)
 *   bound      = scale * q_norm_max * k_norm_max
 *                (Cauchy-Schwarz: >= scale * q_i . (k_j - mu) for all i, j)
 *   gap_est    = scale * q_norm_max * (k_norm_max + c_max)
 *                (>= bound minus the largest live logit of every row)
 *   eligible   = gap_est <= gap_threshold_nats and the key mean finite (1)
 *                or not (0)
 * 32 bytes, naturally aligned.
 */
typedef struct fsattn_head_bound {
  float q_norm_max;
  float k_norm_max;
  float c_max;
  float bound;
  float gap_est;
  int32_t eligible;
  int32_t pad[2];
} fsattn_head_bound;

/* fsattn_forward flags. */
enum {
  FSATTN_MODE_AUTO = 0,          /* fixed shift on eligible heads, online elsewhere */
  FSATTN_MODE_FORCE_ONLINE = 1,  /* online softmax on every head */
  FSATTN_MODE_FORCE_FIXED = 2,   /* fixed shift on every head (testing; an
                                    ineligible head may underflow to 0/0) */
  FSATTN_SHIFT_PER_ROW = 4       /* fixed shift scale*(|q_i|*k_norm_max + q_i.mu)
                                    instead of bound + scale*q_i.mu */
};
/* Optional launch-shape overrides in the flags word (0 = library choice),
 * bf16 inputs only: bits 8..11 waves per workgroup (2, 4 or 8), bits
 * 12..15 query rows per wave divided by 16 (1..4; the library's own
 * choice divides tokens_per_frame, an explicit one need not: a frame's
 * last wave then also computes rows past the frame's end, on the frame's
 * last query row, and stores only its live rows), bits 16..19 keys per
 * pipeline step divided by 16 (2 or 4), bits 20..23 K/V staging buffers in
 * the ring (2, 3 or 4; 3 and 4 with 32-key steps only). An override that is not built or does not fit
 * the geometry returns FSATTN_ERR_UNSUPPORTED. */
#define FSATTN_FLAG_WAVES(n) ((uint32_t)(n) << 8)
#define FSATTN_FLAG_ROWS16(m) ((uint32_t)(m) << 12)
#define FSATTN_FLAG_KSTEP16(s) ((uint32_t)(s) << 16)
#define FSATTN_FLAG_RING(b) ((uint32_t)(b) << 20)
/* How the query tiles are dealt to the XCDs, bits 24..27 (bf16 inputs
 * only): 0 = library choice, 1..14 = chunks of 2^(v-1) consecutive tiles
 * of one (frame, head) group, 15 = whole groups. The results do not depend
 * on it (every tile is computed the same way wherever it runs). */
#define FSATTN_FLAG_DEAL(v) ((uint32_t)(v) << 24)

#define FSATTN_DEFAULT_GAP_NATS 30.0f

/*
 * Plan size ("Deleting the Mask", Fig. 3: with blocks that divide the frame
 * span, each query frame's live key blocks are whole frames of blocks):
 * number of query blocks (seq_len / block_q) and number of live (query
 * block, key block) pairs, nnz = sum_f |L(f)| * (T/block_q) * (T/block_k),
 * where L(f) is the set of frames query frame f sees. Sizes the arrays of
 * fsattn_plan / fsattn_plan_device. Host only. Errors: INVALID_ARGUMENT
 * (null pointer), BLOCK_GEOMETRY.
 */
fsattn_status fsattn_plan_size(const fsattn_mask *m, int64_t *num_q_blocks, int64_t *nnz);

/*
 * The block plan ("Deleting the Mask": blocks that divide the frame span
 * are full or empty, and the reference frame's blocks are just more full
 * blocks of the same pass). Writes CSR arrays into caller-owned HOST
 * memory: row_ptr[num_q_blocks + 1] with row_ptr[0] = 0, and col_idx[nnz]
 * holding, for each query block in order, its live key blocks in
 * ascending order. The plan depends on the mask only and is shared by
 * every batch and head. Host only, deterministic, bit-exact.
 * Errors: INVALID_ARGUMENT, BLOCK_GEOMETRY, BUFFER_TOO_SMALL.
 */
fsattn_status fsattn_plan(const fsattn_mask *m, int32_t *row_ptr, int64_t row_ptr_len,
                          int32_t *col_idx, int64_t col_idx_len);

/*
 * The same plan as fsattn_plan, element for element, written by a GPU
 * kernel into caller-owned DEVICE memory (row_ptr[num_q_blocks + 1],
 * col_idx[nnz]), so that a pipeline needs no host-to-device copy of it.
 * The lengths are those of the device buffers. Validation is on the host
 * and identical to fsattn_plan's; asynchronous on hip_stream.
 * Errors: INVALID_ARGUMENT, BLOCK_GEOMETRY, UNSUPPORTED (nnz > INT32_MAX),
 * BUFFER_TOO_SMALL, HIP.
 */
fsattn_status fsattn_plan_device(void *hip_stream, const fsattn_mask *m, int32_t *row_ptr,
                                 int64_t row_ptr_len, int32_t *col_idx, int64_t col_idx_len);

/* Bytes of device workspace fsattn_head_bounds (and fsattn_produce) needs
 * for this shape and mask ("Unchaining the Softmax": the per-chunk partial
 * key sums and norm maxima from which the per-head mean, norm maxima and
 * window term are reduced); 0 if the arguments are invalid. */
size_t fsattn_head_bounds_workspace_bytes(const fsattn_shape *s, const fsattn_mask *m);

/*
 * Per-head bounds and eligibility ("Unchaining the Softmax": mean-centred
 * keys, norm maxima, Cauchy-Schwarz bound, per-head eligibility; the bound
 * audit for windowed masks gives c_max). Reads Q and K (device), writes
 * key_mean[B*H*head_dim] (fp32, device; the mean over all N keys of each
 * head) and rec[B*H] (device), using the caller's device workspace
 * (>= fsattn_head_bounds_workspace_bytes). Reductions run in a fixed order
 * without atomics: results are bitwise reproducible. scale > 0;
 * gap_threshold_nats >= 0. Asynchronous on hip_stream.
 * Inputs are meant to be finite. If they are not, the effect stays in the
 * head and, through fsattn_forward, in the rows that touch the value: the
 * norm maxima skip NaN (a NaN query row leaves the record as if the row
 * were absent; that row's output is NaN), and a head whose key mean is not
 * finite (a non-finite key) is marked not eligible, so the online path
 * confines the damage to the rows that attend to that key.
 * Errors: INVALID_ARGUMENT, BLOCK_GEOMETRY, UNSUPPORTED,
 * BUFFER_TOO_SMALL (workspace), HIP.
 */
fsattn_status fsattn_head_bounds(void *hip_stream, const fsattn_shape *s, const fsattn_mask *m,
                                 fsattn_tensor q, fsattn_tensor k, float scale,
                                 float gap_threshold_nats, float *key_mean,
                                 fsattn_head_bound *rec, void *workspace, size_t workspace_bytes);

/*
 * fsattn_head_bounds without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same kernels and the same
 * results, bit for bit, with the workspace in a device-resident array of
 * fsattn_head_bounds_noalloc_max_workspace() bytes (4 MiB) that the library
 * holds on each device it runs on until the process ends. Calls no
 * allocating routine. Arguments and errors are those of fsattn_head_bounds,
 * plus BUFFER_TOO_SMALL when fsattn_head_bounds_workspace_bytes() for the
 * shape exceeds that size (e.g. B*H = 16 at 16 frames of 1024 tokens and
 * head_dim 128 needs about 1.2 MiB). Every call on a device shares that
 * device's array, and nothing in it needs to start at zero: calls that
 * overlap on one device (concurrent streams, or threads) race and must be
 * serialised by the caller. The first call on a device looks up the
 * array's address there (FSATTN_ERR_HIP on failure).
 */
fsattn_status fsattn_head_bounds_noalloc(void *hip_stream, const fsattn_shape *s, const fsattn_mask *m,
                                         fsattn_tensor q, fsattn_tensor k, float scale, float gap_threshold_nats,
                                         float *key_mean, fsattn_head_bound *rec);

/* Size in bytes of the device-resident workspace of
 * fsattn_head_bounds_noalloc (the largest workspace it accepts). */
size_t fsattn_head_bounds_noalloc_max_workspace(void);

/*
 * The input-producing chain fused with the bounds ("Layout Is the ABI",
 * Fig. 5: the small operations that make attention's inputs run as one
 * kernel that writes its consumer's layout). Reads Q, K and V through the
 * views q_in, k_in, v_in (any [B,H,N,d] strides, e.g. the token-major
 * output of a QKV projection: stride_n = 3*H*d, stride_h = d); for Q and K
 * applies, per token row and in this order,
 *   RMS normalisation  x <- gamma[h] * x / sqrt(mean(x^2) + eps)
 *   rotary embedding   pair (x[2i], x[2i+1]) of token n rotated by the angle
 *                      with cosine rope_cos[n*d/2 + i], sine rope_sin[...]
 * and writes Q, K and the unchanged V, rounded to s->dtype, through the
 * views q, k, v. gamma_q / gamma_k: device fp32 [H][d], 16-byte aligned,
 * or NULL (that operand is not normalised); eps >= 0. rope_cos / rope_sin:
 * device fp32 [N][d/2], 16-byte aligned, both or neither (NULL: no
 * rotation); the tables carry the positional scheme (1-D or per-axis video
 * positions alike). Inputs and outputs have s->dtype. An output may be the
 * same view as its input (in place); other overlaps are undefined.
 * In the same pass it accumulates the statistics of fsattn_head_bounds on
 * the values it writes, then finishes the bounds: key_mean, rec, scale,
 * gap_threshold_nats and workspace (>= fsattn_head_bounds_workspace_bytes)
 * are as there, and the results equal, bit for bit, fsattn_head_bounds
 * called on the outputs. Asynchronous on hip_stream.
 * Errors: INVALID_ARGUMENT, BLOCK_GEOMETRY, UNSUPPORTED, BUFFER_TOO_SMALL,
 * HIP.
 */
fsattn_status fsattn_produce(void *hip_stream, const fsattn_shape *s, const fsattn_mask *m,
                             fsattn_tensor q_in, fsattn_tensor k_in, fsattn_tensor v_in,
                             const float *gamma_q, const float *gamma_k, float eps,
                             const float *rope_cos, const float *rope_sin,
                             fsattn_tensor q, fsattn_tensor k, fsattn_tensor v, float scale,
                             float gap_threshold_nats, float *key_mean, fsattn_head_bound *rec,
                             void *workspace, size_t workspace_bytes);

/*
 * Attention over the live blocks:
 *   O_i = sum_{j live for i} exp(scale*q_i.k_j - m_i) v_j / sum_j exp(...)
 * in one pass over the plan's key blocks ("Deleting the Mask"), with m_i
 * either the precomputed per-row shift (fixed path, "Unchaining the
 * Softmax", Fig. 4 lower) or the running max (online path, Fig. 4 upper),
 * chosen per head from rec[].eligible and flags. QK^T and PV run on bf16
 * MFMA with fp32 accumulation for bf16 inputs (P is rounded to bf16 for
 * PV); fp32 inputs are computed in fp32 throughout.
 *
 * row_ptr/col_idx: DEVICE copies of fsattn_plan's output for the same mask
 * (nnz entries); the kernel relies on all query blocks of a frame sharing
 * one list, which fsattn_plan guarantees. key_mean/rec: fsattn_head_bounds'
 * output for the same Q/K and scale (needed by the fixed path; may be NULL
 * only with FSATTN_MODE_FORCE_ONLINE; key_mean 16-byte aligned). o: output [B,H,N,d] of o_dtype
 * (the input dtype, or FSATTN_F32). lse: optional device [B*H*N] fp32
 * log-sum-exp (natural log) per row, or NULL. Asynchronous on hip_stream;
 * deterministic (no atomics).
 * Errors: INVALID_ARGUMENT (incl. nnz not matching the mask), BLOCK_GEOMETRY,
 * UNSUPPORTED, HIP.
 */
fsattn_status fsattn_forward(void *hip_stream, const fsattn_shape *s, const fsattn_mask *m,
                             const int32_t *row_ptr, const int32_t *col_idx, int64_t nnz,
                             fsattn_tensor q, fsattn_tensor k, fsattn_tensor v, fsattn_tensor o,
                             int32_t o_dtype, const float *key_mean, const fsattn_head_bound *rec,
                             float scale, uint32_t flags, float *lse);

/*
 * Launch shape fsattn_forward would use for these arguments (host only):
 * waves per workgroup, query rows per wave, keys per pipeline step, query
 * tiles (one workgroup each; the bf16 grid adds up to 7 idle ids so that
 * every XCD gets whole rounds) and dynamic LDS bytes per workgroup. Any
 * output pointer may be NULL. Errors: as fsattn_forward's host validation.
 */
fsattn_status fsattn_forward_launch_info(const fsattn_shape *s, const fsattn_mask *m, uint32_t flags,
                                         int32_t *waves, int32_t *rows_per_wave, int32_t *key_step,
                                         int64_t *workgroups, int32_t *lds_bytes);

/*
 * Comparator (not part of the attention path): the same attention computed
 * the way "Deleting the Mask" describes the prior art, so that the gain of
 * frame-aligned blocks and the single pass can be measured on this device.
 * The sequence is tiled in 128-token query and key tiles (padded at its
 * end), not aligned to frames; a first pass covers each row's window, a
 * second pass the reference frame for the rows whose window does not hold
 * it; key tiles that are only partly live for a query tile evaluate a
 * per-element frame predicate; both passes use the online softmax and write
 * normalised fp32 rows and log-sum-exps to the workspace, and a third kernel
 * merges them into o. bf16 inputs only (same MFMA, LDS staging and copies as
 * fsattn_forward's default launch); block_q/block_k of the mask are not
 * used, and global reference frames (ref_queries_global = 1) or more than
 * one reference frame (ref_count > 1) are UNSUPPORTED. workspace: DEVICE memory, 16-byte aligned, >=
 * fsattn_prior_art_workspace_bytes(). Asynchronous on hip_stream.
 * Errors: INVALID_ARGUMENT, BLOCK_GEOMETRY, UNSUPPORTED, BUFFER_TOO_SMALL,
 * HIP.
 */
fsattn_status fsattn_prior_art_forward(void *hip_stream, const fsattn_shape *s, const fsattn_mask *m,
                                       fsattn_tensor q, fsattn_tensor k, fsattn_tensor v, fsattn_tensor o,
                                       int32_t o_dtype, float scale, void *workspace, size_t workspace_bytes);

/* Workspace bytes of fsattn_prior_art_forward (0 for invalid arguments or
 * non-bf16 inputs). */
size_t fsattn_prior_art_workspace_bytes(const fsattn_shape *s, const fsattn_mask *m);

/*
 * Measurement aid (not part of the attention path): a reference rate for
 * the matrix unit. Launches `workgroups` workgroups of 4 waves that each
 * run `iters` rounds of 8 independent v_mfma_f32_16x16x32_bf16 (the forward
 * kernel's instruction) on register operands, with no memory traffic, and
 * write one float per workgroup to sink (DEVICE memory, >= workgroups
 * floats; the values carry no meaning). *flops (host, may be NULL)
 * receives the launch's multiply-add count x 2. Timing the launch on the
 * stream gives the bf16 MFMA rate the device reaches at the clock it holds
 * under a pure matrix load. Errors: INVALID_ARGUMENT (workgroups outside
 * [1, 2^20], iters < 1, NULL sink), HIP.
 */
fsattn_status fsattn_mfma_probe(void *hip_stream, int32_t workgroups, int32_t iters, float *sink,
                                int64_t *flops);

/* Static description of a status code. */
const char *fsattn_status_string(fsattn_status st);

/* FSATTN_ABI_VERSION of the built library. */
int fsattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FSATTN_H */
