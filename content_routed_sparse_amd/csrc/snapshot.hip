// Session snapshot and restore of the cache state (release post, on keeping the cache: sessions
// saved to and restored from disk; the InfiniteKV post's hashed receipts and SHA-256 checks).
//
// The image is header | payload | digest levels | root (layout in include/routed_attn.h).  On the
// device it is built by three kinds of launch, all stream-ordered and allocation-free:
//  * write_words: the header's 64-bit words, passed by value;
//  * copy_segments: up to kSegs contiguous byte ranges per launch (the live rows of K and V of
//    each (sequence, kv head), the complete span means, the running sums), 16 bytes per lane,
//    non-temporal; the 8-bit cache's row scales 4 bytes per lane (a scale run need not start on
//    16 bytes in the cache), and the zero padding after each run; restore runs the same kernel
//    the other way, behind a guard word so that a failed check leaves the caller's cache untouched;
//  * sha_chunks: one lane per chunk (4096 bytes of data, or a group of 16 digests of the level
//    below) computes its SHA-256 (the blocks in a row, the next block's four 16-byte loads issued
//    before the current block's rounds) and either stores the digest or compares it with the
//    stored one (atomicMin of the chunk's offset on a mismatch).  The levels run one launch
//    each; their inputs are the previous launch's output.
// Hashing is bound by the vector ALU: 1,416 VALU instructions per 64-byte block.
#include "common.h"
#include "sha256.h"
#include "snapshot_kernels.h"

namespace ra {
namespace {

constexpr int kHashThreads = 256;

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte loads and stores marked non-temporal: every byte is touched once per call.
__device__ __forceinline__ uint4 ld_once(const uint4 *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_once(uint4 *p, const uint4 &v) {
    const u32x4_t x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t *>(p));
}

__global__ void __launch_bounds__(kHashThreads) sha_chunks(const uint8_t *__restrict__ src, uint64_t n_bytes,
                                                           uint32_t chunk, uint8_t *__restrict__ dig,
                                                           uint64_t n_chunks, int compare,
                                                           unsigned long long *__restrict__ bad, uint64_t src_offset) {
    using namespace sha256;
    const uint64_t c = (uint64_t)blockIdx.x * kHashThreads + threadIdx.x;
    if (c >= n_chunks) return;
    const uint64_t lo = c * chunk;
    const uint32_t len = (uint32_t)(n_bytes - lo < (uint64_t)chunk ? n_bytes - lo : (uint64_t)chunk);
    const uint4 *p = reinterpret_cast<const uint4 *>(src + lo);
    uint32_t st[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) st[i] = kInit[i];
    const uint32_t full = len / 64;  // complete 64-byte blocks (len is a multiple of 16)
    uint4 nx[4];
    if (full > 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) nx[i] = ld_once(p + i);
    }
    for (uint32_t blk = 0; blk < full; ++blk) {
        uint32_t w[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[4 * i] = bswap(nx[i].x);
            w[4 * i + 1] = bswap(nx[i].y);
            w[4 * i + 2] = bswap(nx[i].z);
            w[4 * i + 3] = bswap(nx[i].w);
        }
        if (blk + 1 < full) {
#pragma unroll
            for (int i = 0; i < 4; ++i) nx[i] = ld_once(p + 4 * (blk + 1) + i);
        }
        compress(st, w);
    }
    // last block: the remaining 0, 16, 32 or 48 bytes, the 1 bit, zeros, the bit length
    {
        const uint32_t rem = len % 64;
        uint32_t w[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) w[i] = 0u;
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            if (16u * (i + 1) <= rem) {
                const uint4 v = p[4 * full + i];
                w[4 * i] = bswap(v.x);
                w[4 * i + 1] = bswap(v.y);
                w[4 * i + 2] = bswap(v.z);
                w[4 * i + 3] = bswap(v.w);
            }
        }
        const uint32_t pw = rem / 4;
#pragma unroll
        for (int i = 0; i < 13; i += 4)  // pw is 0, 4, 8 or 12
            if ((uint32_t)i == pw) w[i] = 0x80000000u;
        w[14] = 0u;  // len < 2^29 bytes
        w[15] = len * 8u;
        compress(st, w);
    }
    uint4 d0 = make_uint4(bswap(st[0]), bswap(st[1]), bswap(st[2]), bswap(st[3]));
    uint4 d1 = make_uint4(bswap(st[4]), bswap(st[5]), bswap(st[6]), bswap(st[7]));
    uint4 *out = reinterpret_cast<uint4 *>(dig + 32 * c);
    if (!compare) {
        out[0] = d0;
        out[1] = d1;
    } else {
        const uint4 s0 = out[0], s1 = out[1];
        const bool same = s0.x == d0.x && s0.y == d0.y && s0.z == d0.z && s0.w == d0.w && s1.x == d1.x &&
                          s1.y == d1.y && s1.z == d1.z && s1.w == d1.w;
        if (!same) atomicMin(bad, (unsigned long long)(src_offset + lo));
    }
}

__global__ void __launch_bounds__(256) copy_segments(SegmentBatch sb, const unsigned long long *guard) {
    if (guard != nullptr && *guard != ~0ull) return;
    const Segment s = sb.seg[blockIdx.y];
    const uint64_t step = (uint64_t)gridDim.x * 256, i0 = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (s.mode == kSegCopy16) {
        const uint4 *src = reinterpret_cast<const uint4 *>(s.src);
        uint4 *dst = reinterpret_cast<uint4 *>(s.dst);
        for (uint64_t i = i0; i < s.n; i += step) st_once(dst + i, ld_once(src + i));
    } else if (s.mode == kSegCopy4) {
        const uint32_t *src = reinterpret_cast<const uint32_t *>(s.src);
        uint32_t *dst = reinterpret_cast<uint32_t *>(s.dst);
        for (uint64_t i = i0; i < s.n; i += step) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
    } else {
        uint32_t *dst = reinterpret_cast<uint32_t *>(s.dst);
        for (uint64_t i = i0; i < s.n; i += step) dst[i] = 0u;
    }
}

__global__ void __launch_bounds__(256) write_words(uint64_t *dst, WordBatch wb) {
    if ((int)threadIdx.x < wb.n) dst[threadIdx.x] = wb.v[threadIdx.x];
}

}  // namespace

hipError_t launch_copy_segments(const SegmentBatch &sb, const unsigned long long *guard, hipStream_t st) {
    if (sb.n == 0) return hipSuccess;
    uint64_t most = 0;
    for (int i = 0; i < sb.n; ++i) most = sb.seg[i].n > most ? sb.seg[i].n : most;
    if (most == 0) return hipSuccess;
    uint64_t gx = (most + 255) / 256;
    if (gx > 4096) gx = 4096;
    hipLaunchKernelGGL(copy_segments, dim3((unsigned)gx, (unsigned)sb.n), dim3(256), 0, st, sb, guard);
    return hipGetLastError();
}

hipError_t launch_write_words(uint64_t *dst, const WordBatch &wb, hipStream_t st) {
    if (wb.n == 0) return hipSuccess;
    hipLaunchKernelGGL(write_words, dim3(1), dim3(256), 0, st, dst, wb);
    return hipGetLastError();
}

hipError_t launch_sha_chunks(const uint8_t *src, uint64_t n_bytes, uint64_t chunk, uint8_t *dig, bool compare,
                             unsigned long long *bad, uint64_t src_offset, hipStream_t st) {
    const uint64_t n = (n_bytes + chunk - 1) / chunk;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(sha_chunks, dim3((unsigned)((n + kHashThreads - 1) / kHashThreads)), dim3(kHashThreads), 0, st,
                       src, n_bytes, (uint32_t)chunk, dig, n, compare ? 1 : 0, bad, src_offset);
    return hipGetLastError();
}

hipError_t launch_fill_u64(unsigned long long *dst, unsigned long long v, hipStream_t st) {
    WordBatch wb;
    wb.n = 1;
    wb.v[0] = v;
    return launch_write_words(reinterpret_cast<uint64_t *>(dst), wb, st);
}

}  // namespace ra
