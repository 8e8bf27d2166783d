// Masked vocab-parallel embedding lookup of one shard.
//
// Method: MiniMind-Tron "5 Vocab Parallelism", 5.2.1 (and Figure 1 of the
// interview note "Vocab parallelism"): an id inside the shard's interval
// [start, end) selects local row id - start; every other id yields a zero row,
// so the T shards' outputs sum to the dense lookup.
//
// HBM-bound: the output rows are a streaming write of 16-byte stores (plain
// stores measured ~15% faster than non-temporal ones here), owned shard rows are
// read with 16-byte loads so that repeated (Zipf-frequent) ids hit in L2 / MALL,
// and off-shard rows read nothing.  One wave per output row: the row's id is a
// wave-uniform scalar load, so the owned / zero decision is a scalar branch, and
// each lane keeps up to eight 16-byte loads or stores in flight.
#include "common.hpp"
#include "launch.hpp"

namespace vp {

namespace {

constexpr int kEmbThreads = 256;
constexpr int kEmbUnroll = 8;   // 16-byte chunks per lane in flight

__global__ __launch_bounds__(kEmbThreads) void embed_kernel(const int64_t *__restrict__ ids,
                                                            int64_t n,
                                                            const uint16_t *__restrict__ w,
                                                            int64_t start, int64_t end, int64_t h,
                                                            uint16_t *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * (kEmbThreads / 64);
    const int64_t chunks = h >> 3;   // 16-byte chunks per row
    for (int64_t row = (int64_t)blockIdx.x * (kEmbThreads / 64) + wave_in_block; row < n;
         row += nwaves) {
        const int64_t id = ids[row];   // uniform: one scalar load per wave
        u32x4 *dst = (u32x4 *)(out + row * h);
        if (id >= start && id < end) {
            const u32x4 *src = (const u32x4 *)(w + (id - start) * h);
            for (int64_t c0 = lane; c0 < chunks; c0 += kEmbUnroll * 64) {
                u32x4 v[kEmbUnroll];
#pragma unroll
                for (int k = 0; k < kEmbUnroll; ++k)
                    if (c0 + 64 * k < chunks) v[k] = src[c0 + 64 * k];
#pragma unroll
                for (int k = 0; k < kEmbUnroll; ++k)
                    if (c0 + 64 * k < chunks) dst[c0 + 64 * k] = v[k];
            }
        } else {
            const u32x4 z = {0u, 0u, 0u, 0u};
            for (int64_t c = lane; c < chunks; c += 64) dst[c] = z;
        }
    }
}

}  // namespace

hipError_t launch_embed(const int64_t *ids, int64_t n, const uint16_t *w, int64_t start,
                        int64_t end, int64_t h, uint16_t *out, hipStream_t stream) {
    // one wave per row (grid-stride beyond 2^20 workgroups)
    int64_t blocks = ceil_div(n, kEmbThreads / 64);
    if (blocks > (1 << 20)) blocks = 1 << 20;
    hipLaunchKernelGGL(embed_kernel, dim3((unsigned)blocks), dim3(kEmbThreads), 0, stream, ids, n,
                       w, start, end, h, out);
    return hipGetLastError();
}

}  // namespace vp
