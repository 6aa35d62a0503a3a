// Internal launch interface of the cold-retrieval kernels (cold.hip) for the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace ra {

constexpr int kMaxCold = 128;      // largest top_k_cold
constexpr int kMergeTiles = 4096;  // scan tiles per row (of cold_tile_positions(G) positions each)

struct SigArgs {  // signatures of rows [old_len[b], new_len[b]) of a K cache
    const void *k;
    uint32_t *sig;  // [B][Hkv][cap][d / 32] words
    const int64_t *old_len, *new_len;
    int dtype, d, B, Hkv;
    int64_t cap, max_new;
};

// Cold positions per scan tile for G query heads per kv head; scan tiles per (row, kv head) for
// rows up to max_pos; and the candidate workspace they fill.
int cold_tile_positions(int G);
int cold_tiles(int64_t max_pos, int H, int G);
size_t cold_workspace_bytes(const RowArgs &a, int H, int kc);

hipError_t launch_signatures(const SigArgs &a, hipStream_t st);
hipError_t launch_cold_select(const RowArgs &a, const uint32_t *sig, int H, int kc, int32_t *sel, void *ws,
                              hipStream_t st);
hipError_t launch_cold_attn(const RowArgs &a, const void *K, const void *V, const int32_t *sel, int H, int kc,
                            float *out, hipStream_t st);

}  // namespace ra
