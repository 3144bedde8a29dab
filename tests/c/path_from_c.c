/* The whole attention path from plain C99 with the HIP runtime's C API and
 * no other framework: device plan, head bounds, forward, on the null stream.
 *
 * usage: path_from_c DIR B H F T d wb wa ref bq bk
 * DIR holds q.bin, k.bin, v.bin: bf16 bit patterns (uint16) of [B, H, N, d],
 * N = F * T. Writes DIR/o.bin (bf16 bit patterns, [B, H, N, d]) and
 * DIR/rec.bin (the B * H fsattn_head_bound records). Exit status 0 on
 * success; on any error prints the failing call and its status. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fsattn.h"

#define HIP_OK(call)                                                    \
  do {                                                                  \
    hipError_t e_ = (call);                                             \
    if (e_ != hipSuccess) {                                             \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_)); \
      return 1;                                                         \
    }                                                                   \
  } while (0)

#define FS_OK(call)                                                                     \
  do {                                                                                  \
    fsattn_status s_ = (call);                                                          \
    if (s_ != FSATTN_OK) {                                                              \
      fprintf(stderr, "%s failed: %d (%s)\n", #call, (int)s_, fsattn_status_string(s_)); \
      return 1;                                                                         \
    }                                                                                   \
  } while (0)

static int io(const char *dir, const char *name, void *buf, size_t bytes, int write) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, write ? "wb" : "rb");
  if (!f) return 1;
  const size_t n = write ? fwrite(buf, 1, bytes, f) : fread(buf, 1, bytes, f);
  fclose(f);
  return n == bytes ? 0 : 1;
}

int main(int argc, char **argv) {
  if (argc != 12) {
    fprintf(stderr, "usage: %s DIR B H F T d wb wa ref bq bk\n", argv[0]);
    return 2;
  }
  const char *dir = argv[1];
  fsattn_shape s;
  fsattn_mask m;
  memset(&s, 0, sizeof s);
  memset(&m, 0, sizeof m);
  s.batch = atoi(argv[2]);
  s.heads = atoi(argv[3]);
  m.num_frames = atoi(argv[4]);
  m.tokens_per_frame = atoi(argv[5]);
  s.head_dim = atoi(argv[6]);
  m.window_before = atoi(argv[7]);
  m.window_after = atoi(argv[8]);
  m.ref_frame = atoi(argv[9]);
  m.block_q = atoi(argv[10]);
  m.block_k = atoi(argv[11]);
  s.seq_len = m.num_frames * m.tokens_per_frame;
  s.dtype = FSATTN_BF16;
  const int64_t BH = (int64_t)s.batch * s.heads, N = s.seq_len, d = s.head_dim;
  const size_t elems = (size_t)(BH * N * d), bytes = elems * 2;

  unsigned short *host = malloc(bytes);
  void *dq, *dk, *dv, *dout;
  HIP_OK(hipMalloc(&dq, bytes));
  HIP_OK(hipMalloc(&dk, bytes));
  HIP_OK(hipMalloc(&dv, bytes));
  HIP_OK(hipMalloc(&dout, bytes));
  const char *names[3] = {"q.bin", "k.bin", "v.bin"};
  void *dst[3] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    if (io(dir, names[i], host, bytes, 0)) {
      fprintf(stderr, "cannot read %s/%s\n", dir, names[i]);
      return 1;
    }
    HIP_OK(hipMemcpy(dst[i], host, bytes, hipMemcpyHostToDevice));
  }

  /* plan, written on the device */
  int64_t nqb = 0, nnz = 0;
  FS_OK(fsattn_plan_size(&m, &nqb, &nnz));
  int32_t *row_ptr, *col_idx;
  HIP_OK(hipMalloc((void **)&row_ptr, sizeof(int32_t) * (size_t)(nqb + 1)));
  HIP_OK(hipMalloc((void **)&col_idx, sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1)));
  FS_OK(fsattn_plan_device(NULL, &m, row_ptr, nqb + 1, col_idx, nnz));

  /* bounds */
  const size_t ws_bytes = fsattn_head_bounds_workspace_bytes(&s, &m);
  if (ws_bytes == 0) {
    fprintf(stderr, "fsattn_head_bounds_workspace_bytes rejected the shape\n");
    return 1;
  }
  void *ws;
  float *key_mean;
  fsattn_head_bound *rec;
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMalloc((void **)&key_mean, sizeof(float) * (size_t)(BH * d)));
  HIP_OK(hipMalloc((void **)&rec, sizeof(fsattn_head_bound) * (size_t)BH));
  fsattn_tensor t[4];
  void *ptrs[4] = {dq, dk, dv, dout};
  for (int i = 0; i < 4; ++i) {
    t[i].data = ptrs[i];
    t[i].stride_b = s.heads * N * d;
    t[i].stride_h = N * d;
    t[i].stride_n = d;
  }
  const float scale = 1.0f / sqrtf((float)d);
  FS_OK(fsattn_head_bounds(NULL, &s, &m, t[0], t[1], scale, FSATTN_DEFAULT_GAP_NATS, key_mean, rec, ws, ws_bytes));

  /* forward */
  FS_OK(fsattn_forward(NULL, &s, &m, row_ptr, col_idx, nnz, t[0], t[1], t[2], t[3], FSATTN_BF16, key_mean, rec,
                       scale, FSATTN_MODE_AUTO, NULL));
  HIP_OK(hipDeviceSynchronize());

  HIP_OK(hipMemcpy(host, dout, bytes, hipMemcpyDeviceToHost));
  fsattn_head_bound *hrec = malloc(sizeof(fsattn_head_bound) * (size_t)BH);
  HIP_OK(hipMemcpy(hrec, rec, sizeof(fsattn_head_bound) * (size_t)BH, hipMemcpyDeviceToHost));
  if (io(dir, "o.bin", host, bytes, 1) || io(dir, "rec.bin", hrec, sizeof(fsattn_head_bound) * (size_t)BH, 1)) {
    fprintf(stderr, "cannot write the outputs\n");
    return 1;
  }
  hipFree(dq);
  hipFree(dk);
  hipFree(dv);
  hipFree(dout);
  hipFree(row_ptr);
  hipFree(col_idx);
  hipFree(ws);
  hipFree(key_mean);
  hipFree(rec);
  free(host);
  free(hrec);
  printf("ok %lld query blocks, %lld live blocks\n", (long long)nqb, (long long)nnz);
  return 0;
}
