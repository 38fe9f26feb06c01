// Internal: the bf16-MFMA grouped GEMM path (gemm.hip).
#pragma once

#include "common.h"

namespace coli {

struct GemmArgs {
    const WorkItem* items;
    const int32_t* n_items;
    const int32_t* rows_tok;   // token of each slot-list entry
    const int32_t* rows_out;   // output row of each slot-list entry
    int2* tiles;               // (item, first token) per 64-token tile
    int32_t* n_tiles;
    uint16_t* xb;              // [T][H] bf16 activations
    float* sx;                 // [T][H/64] sums of the bf16 activations per 64 columns
    uint16_t* hb;              // [R][I] bf16 intermediate, by output row
    float* sh;                 // [R][I/64] sums of the bf16 intermediate per 64 columns
    float* y_rows;             // [R][H] unweighted expert outputs, by output row
    BlobLayout L;
    int32_t H, I, group;
    int32_t gv_max;            // items with at most this many tokens go to the GEMV list (0: none)
    WorkItem* gv_items;        // [max_items] GEMV work list (items in order)
    int32_t* n_gv;
};

// Upper bound of the number of 64-token tiles for `rows` slot-list rows
// spread over at most `max_items` work items.
size_t gemm_tiles_max(int32_t rows, int32_t max_items);

// prep (x -> bf16 + group sums), tile list (and GEMV list), gate/up GEMM, down GEMM.
coli_status launch_mfma_ffn(const GemmArgs& a, const float* x, int32_t T, int32_t max_tiles,
                            hipStream_t stream);

}  // namespace coli
