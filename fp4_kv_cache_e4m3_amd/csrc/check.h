// Parameters of the device-side check of index rows (check.hip).
#pragma once
#include "common.h"

namespace csa2 {

struct CheckParams {
  const int32_t* pool; const int32_t* topk;              // [nq, 2048] (or NULL) and [nq, 512] (or NULL in mode 2)
  const int32_t* nvis; int64_t T;                        // visible positions per query (NULL: all T)
  int32_t mode;                                          // 0 Full outputs, 1 Reindex outputs, 2 Reindex input pool
  uint32_t* bad;                                         // the number of failing rows is added here
};

hipError_t launch_check_index(const CheckParams& p, int nq, hipStream_t st);

}  // namespace csa2
