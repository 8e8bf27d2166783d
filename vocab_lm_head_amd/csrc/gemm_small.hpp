// 128 x 128-tile form of the NT GEMM (C[m, n] = sum_k A[m, k] B[n, k], fp32 out[n, m] = C[m, n])
// for the two gradient products when their 256 x 256 tiles would leave most CUs idle and
// their K loops are short: there a K split pays for its fp32 partials and their sum more
// than it gains, while 128 x 128 tiles fill the chip in one round with no partials.
//
// Workgroup: 8 waves.  Wave w computes the 64 x 64 sub-tile (w & 3) of the tile over K half
// (w >> 2) of every 64-wide K step (v_mfma_f32_16x16x32_bf16, 16 per wave per step).  The two
// halves' accumulators are added through LDS at the end, half 0's plus half 1's, so the
// result does not depend on timing.  With 2 waves per SIMD one wave's MFMAs run while the
// other's LDS reads are in flight.
//
// Pipeline: 3 LDS stages of [128 x 64] A and [128 x 64] B (3 x 32 KiB, the same swizzled
// layout as the 256 x 256 kernel); step k lives in stage k % 3 and its loads are issued two
// steps ahead, each wave loading 16 rows of A and 16 of B.  One workgroup barrier per step
// orders everything:
//   - the loads of step k + 2 go into the stage of step k - 1; they are issued after the
//     barrier that follows every wave's wait for its own reads of step k - 1;
//   - step k + 1 is read after the barrier that follows every wave's wait for its own loads
//     of step k + 1.
// So no wave's loads can overwrite rows another wave is still reading, whatever the waves'
// relative progress.
//
// Rows past M / N and K chunks past K read as zeros, as in the 256 x 256 kernel.
#pragma once

#include <type_traits>

#include "gemm.hpp"

namespace vp {

constexpr int kSBM = 128, kSBN = 128;
constexpr int kSWaves = 8;
constexpr int kSThreads = 64 * kSWaves;
constexpr int kSTM = 4, kSTN = 4;               // MFMA tiles per wave (64 x 64)
constexpr int kSStages = 3;
constexpr int kSStage = (kSBM + kSBN) * kBK;    // elements per LDS stage (32 KiB)
constexpr int kSLoads = kSBM / kSWaves / 8;     // load instructions per operand per wave per step
static_assert(kSLoads == 2 && kSBM == kSBN, "each wave loads 16 rows of A and 16 of B per step");

typedef f32x4 SAcc[kSTM][kSTN];

// One product: out[n, m] = C[m, n] for m < M, n < N, over a tiles_m x tiles_n grid.
struct SmallJob {
    Operand A, B;
    int K;
    int tiles_m, tiles_n;
    float *out;
    int64_t ldo;   // multiple of 4, >= M
    int M, N;
    int blocks() const { return tiles_m * tiles_n; }
};

// Two jobs in one launch of blocks0 + blocks(j1) workgroups; workgroups are spread over
// the XCDs in contiguous ranges of the combined tile list (as in tile_of_block), each
// job's tiles walked with m fastest so that an XCD's tiles share B panels in its L2.
__global__ __launch_bounds__(kSThreads, 1) void gemm_nt_small_kernel(SmallJob j0, SmallJob j1,
                                                                     int blocks0, int total) {
    __shared__ __attribute__((aligned(1024))) uint16_t smem[kSStages * kSStage];
    const int bid = blockIdx.x;
    const int q = total >> 3, rr = total & 7;
    const int xcd = bid & 7, local = bid >> 3;
    int pid = xcd * q + min(xcd, rr) + local;
    const bool first = pid < blocks0;
    const SmallJob j = first ? j0 : j1;
    if (!first) pid -= blocks0;
    const int tm = pid % j.tiles_m, tn = pid / j.tiles_m;
    const int m0 = tm * kSBM, n0 = tn * kSBN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = wave >> 2, sub = wave & 3;
    const int wm = sub >> 1, wn = sub & 1;
    const int K = j.K;

    // Global -> LDS, as in the 256 x 256 kernel: one instruction fills 8 rows x 128 B in
    // lane order, lane L fetching logical chunk (L % 8) ^ (row & 7) of row L / 8.
    const int lrow = lane >> 3;
    const int lchunk = (lane & 7) ^ lrow;
    const char *pa = (const char *)(j.A.p + (int64_t)m0 * j.A.ld);
    const char *pb = (const char *)(j.B.p + (int64_t)n0 * j.B.ld);
    const uint32_t bytes_a = resource_bytes((int64_t)(j.A.rows - m0) * j.A.ld * 2);
    const uint32_t bytes_b = resource_bytes((int64_t)(j.B.rows - n0) * j.B.ld * 2);
    const uint32_t row8a = (uint32_t)(8 * j.A.ld * 2), row8b = (uint32_t)(8 * j.B.ld * 2);
    const uint32_t offa = (uint32_t)(((16 * wave + lrow) * j.A.ld + lchunk * 8) * 2);
    const uint32_t offb = (uint32_t)(((16 * wave + lrow) * j.B.ld + lchunk * 8) * 2);
    const int dsta = 16 * wave * kBK, dstb = kSBM * kBK + 16 * wave * kBK;
    auto load_step = [&](int st, int k0) {
        const __amdgpu_buffer_rsrc_t ra =
            __builtin_amdgcn_make_buffer_rsrc((void *)(pa + 2 * k0), (short)0, bytes_a, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rb =
            __builtin_amdgcn_make_buffer_rsrc((void *)(pb + 2 * k0), (short)0, bytes_b, kBufferFlags);
        const bool in = k0 + lchunk * 8 < K;
        const uint32_t oa = in ? offa : kOutOfRange, ob = in ? offb : kOutOfRange;
        uint16_t *s = smem + st * kSStage;
#pragma unroll
        for (int i = 0; i < kSLoads; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(s + dsta + i * 8 * kBK), 16,
                                                     oa + i * row8a, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < kSLoads; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(s + dstb + i * 8 * kBK), 16,
                                                     ob + i * row8b, 0, 0, 0);
    };

    // fragments: lane reads row (lane & 15) of each 16-row tile, logical chunk
    // 4 half + lane / 16 (the wave's 32-wide K half of the step)
    const int fr = lane & 15;
    const int a_off = (wm * 64 + fr) * kBK;
    const int b_off = kSBM * kBK + (wn * 64 + fr) * kBK;
    const int ch = ((4 * half + (lane >> 4)) ^ (fr & 7)) * 8;
    struct Frag {
        bf16x8 a[kSTM];
        bf16x8 b[kSTN];
    };
    auto read_step = [&](int st, Frag &f) {
        const uint16_t *buf = smem + st * kSStage;
#pragma unroll
        for (int i = 0; i < kSTM; ++i) f.a[i] = *(const bf16x8 *)&buf[a_off + i * 16 * kBK + ch];
#pragma unroll
        for (int jj = 0; jj < kSTN; ++jj) f.b[jj] = *(const bf16x8 *)&buf[b_off + jj * 16 * kBK + ch];
    };
    SAcc acc;
#pragma unroll
    for (int i = 0; i < kSTM; ++i)
#pragma unroll
        for (int jj = 0; jj < kSTN; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mma = [&](const Frag &f) {
#pragma unroll
        for (int i = 0; i < kSTM; ++i)
#pragma unroll
            for (int jj = 0; jj < kSTN; ++jj)
                acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[jj], acc[i][jj], 0, 0, 0);
    };

    // loads of one step per wave, and the count that may stay in flight while the next
    // step is awaited (the one step issued after it)
    constexpr int kStepLoads = 2 * kSLoads;
    constexpr int kAhead = (kSStages - 2) * kStepLoads;
    const int KT = (int)ceil_div(K, kBK);
#pragma unroll
    for (int s = 0; s < kSStages - 1; ++s) load_step(s, s * kBK);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(kAhead));   // step 0 has landed
    bare_barrier();
    Frag f[2];
    read_step(0, f[0]);
    int st = 1, lst = kSStages - 1;   // stage of step k + 1; stage the loads of step k + 2 go to
    for (int k = 0; k < KT; k += 2) {
        // two steps per trip, so that the two fragment buffers are named statically
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (k + u < KT) {
                load_step(lst, (k + u + kSStages - 1) * kBK);
                __builtin_amdgcn_s_waitcnt(wait_vmcnt(kAhead));   // step k + u + 1 has landed
                __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);       // this wave's reads of step k + u
                bare_barrier();
                if (k + u + 1 < KT) read_step(st, f[u ^ 1]);
                mma(f[u]);
                __builtin_amdgcn_sched_barrier(0);
                st = st + 1 == kSStages ? 0 : st + 1;
                lst = lst + 1 == kSStages ? 0 : lst + 1;
            }
        }
    }
    // loads past the last step (zeros) may still be landing: drain them before LDS is reused
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    // Half h keeps MFMA row blocks 2h, 2h + 1 of its sub-tile and hands the other two to the
    // other half through LDS: [2 writers][4 sub-tiles][2][4][64 lanes] f32x4 = 64 KiB.
    // Each lane's four accumulator rows are four consecutive m of output row n.
    float *red = (float *)smem;
    const int rsub = 4 * (lane >> 4);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(j.out + (int64_t)n0 * j.ldo + m0, ((int64_t)(j.N - n0) * j.ldo - m0) * 4);
    auto finish = [&](auto keep_c) {
        constexpr int keep = decltype(keep_c)::value, give = 2 - keep;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jj = 0; jj < kSTN; ++jj)
                *(f32x4 *)&red[((((half * 4 + sub) * 2 + i) * kSTN + jj) * 64 + lane) * 4] =
                    acc[give + i][jj];
        __syncthreads();
#pragma unroll
        for (int jj = 0; jj < kSTN; ++jj) {
            const int64_t nl = wn * 64 + 16 * jj + (lane & 15);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const f32x4 other =
                    *(const f32x4 *)&red[(((((half ^ 1) * 4 + sub) * 2 + i) * kSTN + jj) * 64 + lane) * 4];
                // half 0's partial first, on both halves
                const f32x4 v = keep ? other + acc[keep + i][jj] : acc[keep + i][jj] + other;
                const int ml = wm * 64 + 16 * (keep + i) + rsub;
                store16<kStoreDefault>(__builtin_bit_cast(u32x4, v), rs,
                                       m0 + ml < j.M ? (uint32_t)((nl * j.ldo + ml) * 4) : kOutOfRange);
            }
        }
    };
    if (half)
        finish(std::integral_constant<int, 2>());
    else
        finish(std::integral_constant<int, 0>());
}

}  // namespace vp
