// Internal: launchers of the GEMV kernels (gemv_gateup.hip, gemv_down.hip).
#pragma once

#include "common.h"

namespace coli {

// Launch the gate/up kernel on grid (I/16 tiles of 16 rows for mt == 1, else
// I/32 tiles of 32 rows; max_items): h = silu(g) * u of every row it computes,
// as digit planes of 16-element blocks into hplanes / hscale; false if H is
// outside the instantiated range.
bool dispatch_gateup(int mt, int group, dim3 grid, hipStream_t s, const WorkItem* items,
                     const int32_t* n_items, const int32_t* rows_tok, const int32_t* rows_out,
                     const uint32_t* xplanes, const float* xscale, uint32_t* hplanes,
                     float* hscale, int H, int I, const BlobLayout& L, const FusedRoute& fr,
                     const ReadLog& rl);

// Down-matrix rows per wave (4 waves per workgroup). One-token launches take
// 8: twice the workgroups for the same 9 x 6 MB read keep more of it in flight
// (a read-only kernel of that shape: 9.9 us at 8 rows per wave, 10.5 us at 16);
// batches take 16, which shares each wave's activation blocks over more rows.
constexpr int down_rows_per_wave(int mt) { return mt == 1 ? 8 : 16; }

// Launch the down kernel on grid (ceil(H / (4 * down_rows_per_wave(mt))), max_items) into
// y_rows, reading the h blocks that the gate/up pass wrote. False if I is outside
// the instantiated range.
bool dispatch_down(int mt, int group, dim3 grid, hipStream_t s, const WorkItem* items,
                   const int32_t* n_items, const int32_t* rows_out, const uint32_t* hplanes,
                   const float* hscale, float* y_rows, int H, int I, const BlobLayout& L,
                   const ReadLog& rl);

}  // namespace coli
