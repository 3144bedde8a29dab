/* A plain C99 caller of libfsattn.so's host entry points: the header must
 * compile as C and the library must link and run without C++ or Python.
 * Prints the ABI version, the plan of the mask given on the command line
 * (num_frames tokens_per_frame window_before window_after ref_frame block_q
 * block_k) as "nqb nnz", then row_ptr and col_idx on one line each, and the
 * status of a geometry error. */
#include <stdio.h>
#include <stdlib.h>

#include "fsattn.h"

int main(int argc, char **argv) {
  if (argc != 8) {
    fprintf(stderr, "usage: %s F T wb wa ref bq bk\n", argv[0]);
    return 2;
  }
  fsattn_mask m = {0};
  m.num_frames = atoi(argv[1]);
  m.tokens_per_frame = atoi(argv[2]);
  m.window_before = atoi(argv[3]);
  m.window_after = atoi(argv[4]);
  m.ref_frame = atoi(argv[5]);
  m.block_q = atoi(argv[6]);
  m.block_k = atoi(argv[7]);
  printf("abi %d\n", fsattn_abi_version());
  int64_t nqb = 0, nnz = 0;
  fsattn_status st = fsattn_plan_size(&m, &nqb, &nnz);
  if (st != FSATTN_OK) {
    printf("plan_size error %d (%s)\n", (int)st, fsattn_status_string(st));
    return 1;
  }
  int32_t *row_ptr = malloc(sizeof(int32_t) * (size_t)(nqb + 1));
  int32_t *col_idx = malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
  st = fsattn_plan(&m, row_ptr, nqb + 1, col_idx, nnz);
  if (st != FSATTN_OK) {
    printf("plan error %d\n", (int)st);
    return 1;
  }
  printf("%lld %lld\n", (long long)nqb, (long long)nnz);
  for (int64_t i = 0; i <= nqb; ++i) printf("%d%c", row_ptr[i], i == nqb ? '\n' : ' ');
  for (int64_t i = 0; i < nnz; ++i) printf("%d%c", col_idx[i], i + 1 == nnz ? '\n' : ' ');
  fsattn_mask bad = m;
  bad.block_q = 24; /* not a multiple of 16 */
  printf("bad %d\n", (int)fsattn_plan_size(&bad, &nqb, &nnz));
  free(row_ptr);
  free(col_idx);
  return 0;
}
