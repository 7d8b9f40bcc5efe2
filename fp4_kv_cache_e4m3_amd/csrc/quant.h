// Launchers of quant.hip that only the ABI calls (the fp32 ones are declared
// in common.h).
#pragma once
#include "common.h"

namespace csa2 {

// bf16 rows (raw bits): quantised exactly as their fp32 widening would be
hipError_t launch_quantize_bf16(const uint16_t* x, int64_t xs, int64_t rows, int dim, uint8_t* codes,
                                int64_t cs, uint8_t* scales, int64_t ss, hipStream_t st);

}  // namespace csa2
