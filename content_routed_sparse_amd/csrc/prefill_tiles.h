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
    const int4 *tiles;               // (expert, first entry, entries) in XCD order (tile_slot)
    float *records;
    int64_t n_exp, max_tiles, span_slots;
    int NE;
};

// 4-byte words of one partial record: a 16-byte header (m, l, s, 0), then the row's output
// vector: fp32 values o (fp32 inputs), or fp16 values o / (l s) with s a power of two chosen per
// record (bf16 inputs).
__host__ __device__ constexpr int prefill_record_words(int d, bool half) { return 4 + (half ? d / 2 : d); }

// XCD order of the tile descriptors.  The hardware hands block b to XCD b % 8; with Q = ceil(total
// tiles / 8), tile t = x Q + i sits at slot 8 i + x, so that block b runs tile (b % 8) Q + b / 8:
// XCD x takes the contiguous range [x Q, x Q + Q) of the tile list (a span's tiles are consecutive
// there, so they share an L2), and every XCD gets the same number of tiles whatever the launch's
// upper bound on the count.  A slot b holds a tile iff slot_tile(b, total) >= 0.
__host__ __device__ constexpr int64_t tile_slot(int64_t t, int64_t Q) { return 8 * (t % Q) + t / Q; }
__host__ __device__ constexpr int64_t slot_tile(int64_t b, int64_t total) {
    const int64_t Q = (total + 7) / 8, t = (b % 8) * Q + b / 8;
    return b / 8 < Q && t < total ? t : -1;
}
// (checked when compiling: for every count up to 300, slots below 8 Q, each tile in exactly one)
constexpr bool tile_slots_bijective(int64_t max_total) {
    for (int64_t total = 0; total <= max_total; ++total) {
        const int64_t Q = (total + 7) / 8;
        for (int64_t t = 0; t < total; ++t)
            if (tile_slot(t, Q) >= 8 * Q || slot_tile(tile_slot(t, Q), total) != t) return false;
        int64_t held = 0;
        for (int64_t b = 0; b < 8 * Q; ++b) held += slot_tile(b, total) >= 0 ? 1 : 0;
        if (held != total) return false;
    }
    return true;
}
static_assert(tile_slots_bijective(300), "tile slots");

// Entries per tile for this configuration.
int prefill_tile_rows(const RowArgs &a);
hipError_t launch_prefill_tiles(const TileArgs &t, hipStream_t st);

}  // namespace ra
