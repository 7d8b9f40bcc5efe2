// Launcher of the read-rate kernel (rate.hip), called by the ABI only.
#pragma once
#include "common.h"

namespace csa2 {

constexpr int kReadRateWorkgroups = 16384;       // one contiguous chunk each; 4 sink words each
hipError_t launch_read_rate(const void* buf, int64_t bytes, uint32_t* sink, int wgs, hipStream_t st);

}  // namespace csa2
