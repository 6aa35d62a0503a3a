// Internal interface of the prefill tile kernels (span buckets -> partial softmax states).
#pragma once

#include "kernels.h"

namespace ra {

struct TileArgs {
    RowArgs a;
    const void *K, *V;
    const float *ks, *vs;            // row scales of an 8-bit cache (K, V are then E4M3 codes), else null
    const int32_t *tile_off, *list;  // tile count at tile_off[n_exp]; entries
    const int64_t *list_t;           // the entries' row positions
    const int4 *tiles;               // (expert, first entry, entries)
    float *records;
    int64_t n_exp, max_tiles, span_slots;
    int NE;
};

// 4-byte words of one partial record: a 16-byte header (m, l, s, 0), then the row's output
// vector: fp32 values o (fp32 inputs), or fp16 values o / (l s) with s a power of two chosen per
// record (bf16 inputs).
__host__ __device__ constexpr int prefill_record_words(int d, bool half) { return 4 + (half ? d / 2 : d); }

// Entries per tile for this configuration.
int prefill_tile_rows(const RowArgs &a);
hipError_t launch_prefill_tiles(const TileArgs &t, hipStream_t st);

}  // namespace ra
