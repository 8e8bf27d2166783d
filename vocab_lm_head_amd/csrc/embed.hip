// Masked vocab-parallel embedding lookup of one shard.
//
// Method: MiniMind-Tron "5 Vocab Parallelism", 5.2.1 (and Figure 1 of the
// interview note "Vocab parallelism"): an id inside the shard's interval
// [start, end) selects local row id - start; every other id yields a zero row,
// so the T shards' outputs sum to the dense lookup.
//
// HBM-bound: the output rows are a pure streaming write (non-temporal 16-byte
// stores), the shard rows are read with plain 16-byte loads so that repeated
// (Zipf-frequent) ids hit in L2 / MALL; off-shard rows read nothing.  One wave
// per output row at a time, four 1 KiB vectors in flight per lane group.
#include "common.hpp"
#include "launch.hpp"

namespace vp {

namespace {

constexpr int kEmbThreads = 256;

__global__ __launch_bounds__(kEmbThreads) void embed_kernel(const int64_t *__restrict__ ids,
                                                            int64_t n,
                                                            const uint16_t *__restrict__ w,
                                                            int64_t start, int64_t end, int64_t h,
                                                            uint16_t *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = ((int64_t)blockIdx.x * kEmbThreads + threadIdx.x) >> 6;
    const int64_t nwaves = ((int64_t)gridDim.x * kEmbThreads) >> 6;
    const int64_t chunks = h >> 3;   // 16-byte chunks per row
    for (int64_t row = wave; row < n; row += nwaves) {
        const int64_t id = ids[row];
        const bool own = id >= start && id < end;
        const u32x4 *src = (const u32x4 *)(w + (own ? (id - start) : 0) * h);
        u32x4 *dst = (u32x4 *)(out + row * h);
        int64_t c = lane;
        for (; c + 3 * 64 < chunks; c += 4 * 64) {
            u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = v0, v2 = v0, v3 = v0;
            if (own) {
                v0 = src[c];
                v1 = src[c + 64];
                v2 = src[c + 128];
                v3 = src[c + 192];
            }
            __builtin_nontemporal_store(v0, dst + c);
            __builtin_nontemporal_store(v1, dst + c + 64);
            __builtin_nontemporal_store(v2, dst + c + 128);
            __builtin_nontemporal_store(v3, dst + c + 192);
        }
        for (; c < chunks; c += 64) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (own) v = src[c];
            __builtin_nontemporal_store(v, dst + c);
        }
    }
}

}  // namespace

hipError_t launch_embed(const int64_t *ids, int64_t n, const uint16_t *w, int64_t start,
                        int64_t end, int64_t h, uint16_t *out, hipStream_t stream) {
    // enough waves to cover every row once, capped at 32 waves per CU
    const int64_t waves_per_block = kEmbThreads / 64;
    int64_t blocks = ceil_div(n, waves_per_block);
    if (blocks > 256 * 8) blocks = 256 * 8;
    hipLaunchKernelGGL(embed_kernel, dim3((unsigned)blocks), dim3(kEmbThreads), 0, stream, ids, n,
                       w, start, end, h, out);
    return hipGetLastError();
}

}  // namespace vp
