/* A plain C99 consumer of include/mr.h: compiles without HIP headers and exercises the argument
 * checks that return before any HIP call (so it runs on a machine without a GPU). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mr.h"

#define CHECK(cond)                                           \
  do {                                                        \
    if (!(cond)) {                                            \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      return 1;                                               \
    }                                                         \
  } while (0)

int main(void) {
  const void* bufs[2] = {(const void*)0x100000, (const void*)0x200000};
  uint64_t splits[3] = {8, 16, 24};
  int64_t v = -1;
  mr_stream stream = NULL;
  CHECK(mr_version() == 105);
  CHECK(strncmp(mr_status_string(MR_ERR_ALIAS), "MR_ERR_ALIAS", 12) == 0);
  CHECK(mr_allreduce_sum(bufs, 0, 16, MR_BF16, (void*)0x900000, MR_ONESHOT, stream) == MR_ERR_INVALID_ARG);
  CHECK(mr_allreduce_sum(bufs, 2, 16, MR_INT32, (void*)0x900000, MR_ONESHOT, stream) == MR_ERR_DTYPE);
  CHECK(mr_allreduce_sum(bufs, 2, 64, MR_BF16, (void*)0x100002, MR_TWOSHOT, stream) == MR_ERR_ALIAS);
  CHECK(mr_allreduce_sum(NULL, 2, 0, MR_FP32, NULL, MR_ONESHOT, stream) == MR_OK);
  CHECK(mr_allgather_param_contig((const void*)0x100000, 8, 3, splits, 3, MR_FP16, (void*)0x900000, stream) ==
        MR_ERR_INVALID_ARG);
  CHECK(mr_allgather_param_contig((const void*)0x100000, 8, 4, splits, 3, MR_FP16, (void*)0x1002FE, stream) ==
        MR_ERR_ALIAS);
  CHECK(mr_allgather_param_contig_sdma((const void*)0x100000, 8, 3, splits, 3, MR_FP16, (void*)0x900000, stream) ==
        MR_ERR_INVALID_ARG);
  CHECK(mr_allgather_param_contig_sdma((const void*)0x100000, 8, 4, splits, 3, MR_FP16, (void*)0x1002FE, stream) ==
        MR_ERR_ALIAS);
  CHECK(strncmp(mr_status_string(MR_ERR_ENGINE), "MR_ERR_ENGINE", 13) == 0);
  CHECK(mr_allreduce_sum_noalloc(bufs, 0, 16, MR_BF16, (void*)0x900000, MR_TWOSHOT, stream) == MR_ERR_INVALID_ARG);
  CHECK(mr_allreduce_sum_noalloc(bufs, 2, 16, MR_INT32, (void*)0x900000, MR_TWOSHOT, stream) == MR_ERR_DTYPE);
  CHECK(mr_allreduce_sum_noalloc(bufs, 2, MR_NOALLOC_MAX_BYTES / 2 + 1, MR_BF16, (void*)0x90000000, MR_TWOSHOT,
                                 stream) == MR_ERR_WORKSPACE);
  CHECK(mr_allreduce_sum_noalloc(NULL, 2, 0, MR_FP32, NULL, MR_ONESHOT, stream) == MR_OK);
  CHECK(mr_workspace_bytes(8, 1 << 20, MR_BF16) > (2u << 20));
  CHECK(mr_get_option(MR_OPT_TWOSHOT_SYNC, &v) == MR_OK && v == MR_TWOSHOT_SYNC_AUTO);
  CHECK(mr_set_option(MR_OPT_TWOSHOT_SYNC, 7) == MR_ERR_INVALID_ARG);
  CHECK(mr_get_option(MR_OPT_SDMA_CU_BELOW, &v) == MR_OK && v == 1048576);
  CHECK(mr_set_option(MR_OPT_SDMA_CU_BELOW, -1) == MR_ERR_INVALID_ARG);
  CHECK(mr_last_hip_error() == 0);
  printf("c abi ok\n");
  return 0;
}
