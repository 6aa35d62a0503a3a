// Internal launch interface of the snapshot kernels (snapshot.hip) for the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {
// Snapshots: contiguous ranges copied in batches, optionally behind a guard word that must read
// ~0: 16-byte units (16-byte aligned), 4-byte words (4-byte aligned: runs of row scales), or
// 4-byte zero words written to dst (padding; src unused); 64-bit words written from the host by value;
// SHA-256 of each `chunk`-byte piece of src (a multiple of 16 bytes, at most 4096; the last piece
// may be short), stored at dig + 32 * index or compared with it (atomicMin(bad, src_offset +
// the piece's offset) on a mismatch).
enum SegMode : uint32_t { kSegCopy16 = 0, kSegCopy4 = 1, kSegZero4 = 2 };
struct Segment {  // 24 bytes: a batch of kSegs stays within 4 KB of kernel arguments
    const void *src;
    void *dst;
    uint64_t n : 62;    // units of the mode: 16 bytes, or 4 bytes
    uint64_t mode : 2;  // SegMode
};
static_assert(sizeof(Segment) == 24, "Segment is passed by value in batches");
constexpr int kSegs = 128;
struct SegmentBatch {
    Segment seg[kSegs];
    int n;
};
constexpr int kWords = 256;
struct WordBatch {
    uint64_t v[kWords];
    int n;
};
hipError_t launch_copy_segments(const SegmentBatch &sb, const unsigned long long *guard, hipStream_t st);
hipError_t launch_write_words(uint64_t *dst, const WordBatch &wb, hipStream_t st);
hipError_t launch_fill_u64(unsigned long long *dst, unsigned long long v, hipStream_t st);
hipError_t launch_sha_chunks(const uint8_t *src, uint64_t n_bytes, uint64_t chunk, uint8_t *dig, bool compare,
                             unsigned long long *bad, uint64_t src_offset, hipStream_t st);

}  // namespace ra
