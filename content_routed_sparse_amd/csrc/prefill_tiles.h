// Internal interface of the prefill tile kernels (span buckets -> partial softmax states).
#pragma once

#include "kernels.h"

namespace ra {

struct TileArgs {
    RowArgs a;
    const void *K, *V;
    const int32_t *counts, *offsets, *tile_off, *list;
    const int2 *tiles;
    float *records;
    int64_t n_exp, max_tiles, span_slots;
    int NE;
};

// Entries per tile for this configuration.
int prefill_tile_rows(const RowArgs &a);
hipError_t launch_prefill_tiles(const TileArgs &t, hipStream_t st);

}  // namespace ra
