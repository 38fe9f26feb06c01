// Internal: launchers of the GEMV kernels (gemv_gateup.hip, gemv_down.hip).
#pragma once

#include "common.h"

namespace coli {

// Launch the gate/up kernel on grid (I/32, max_items); false if H is outside
// the instantiated range.
bool dispatch_gateup(int mt, int group, dim3 grid, hipStream_t s, const WorkItem* items,
                     const int32_t* n_items, const int32_t* rows_tok, const int32_t* rows_out,
                     const uint32_t* xplanes, const float* xscale, uint32_t* hplanes,
                     float* hscale, int H, int I, const BlobLayout& L);

constexpr int kDownRowsPerWave = 16;
constexpr int kDownRowsPerBlock = 4 * kDownRowsPerWave;

// Launch the down kernel on grid (ceil(H/64), max_items); false if I is
// outside the instantiated range.
bool dispatch_down(int mt, int group, dim3 grid, hipStream_t s, const WorkItem* items,
                   const int32_t* n_items, const int32_t* rows_out, const uint32_t* hplanes,
                   const float* hscale, float* y_rows, int H, int I, const BlobLayout& L);

}  // namespace coli
