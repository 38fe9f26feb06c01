// Expert-level launch of the int4 / int8 quantiser (the other quantiser
// entry points are declared with the rest in common.h).
#pragma once

#include "common.h"

namespace coli {

// An expert's f32 gate [I][H], up [I][H] and down [H][I] matrices into its
// blob regions (gate and up rows at gu_row(r)). Per-row scales: one launch
// for the three matrices when they share the same alignment, else a launch
// for gate and up and one for down; gs64: one launch per matrix.
coli_status launch_quantize_expert(const float* wg, uint8_t* qg, float* sg, const float* wu,
                                   uint8_t* qu, float* su, const float* wd, uint8_t* qd, float* sd,
                                   int64_t H, int64_t I, int32_t group, hipStream_t stream,
                                   int32_t wbits);

}  // namespace coli
