// bf16 x bf16 -> fp32 MFMA GEMM mainloop for gfx950 with a pluggable epilogue.
//
//   C[m, n] = sum_k A[m, k] * B[n, k]        A: [M, K], B: [N, K], both K-contiguous
//
// Every contraction of the LM head is brought to this one form ("NT"):
//   forward / recompute  A = W_r [Vs, H],    B = X   [N, H]    -> C = z^T   (vocab x tokens)
//   dX partial           A = W_r^T [H, Vs],  B = dz  [N, Vs]   -> C = dX^T
//   dW                   A = X^T [H, N],     B = dz^T [Vs, N]  -> C = dW^T
// so each lane's four accumulator rows are four consecutive elements of the
// row-major output it stores (or the four vocabulary rows it reduces over).
//
// Tiling (one workgroup per CU, kWavesM x kWavesN waves of 64 lanes):
//   block tile 256 (M) x 256 (N), K step 64, LDS double buffer 2 x 64 KiB;
//   wave (wm, wn) owns a kWM x kWN sub-tile = kTM x kTN MFMA tiles of
//   v_mfma_f32_16x16x32_bf16 with fp32 accumulators (4 kTM kTN per lane).
// LDS rows are 64 bf16 = 128 B = eight 16-byte chunks; chunk c of row r is
// stored at chunk c ^ (r & 7) so that the 16-lane groups of a fragment read
// (16 consecutive rows, one chunk) hit distinct banks.
// Global -> LDS goes through buffer loads straight into LDS (buffer_load ... lds):
// the loads of K step k+2 are issued in the second half of step k, into the stage
// step k has just finished with.  Operand fragments are double-buffered in
// registers so that the LDS reads of one half K step overlap the MFMAs of the
// other; one barrier per K step.
//
// Rows past M / N read as zeros (outside the buffer resource; the epilogue
// masks them); K chunks past K are zero-filled, so K need only be a multiple
// of 8.  Operands must have 16-byte aligned rows.  Buffer resources are capped
// at 1 GiB (kResourceCap), which holds every byte a 256-row panel's K steps
// reach as long as rows are at most ~2M elements; the C ABI keeps n, h and Vs
// (hence every operand row) at or below 2^20 + 64 elements.
#pragma once

#include "common.hpp"

namespace vp {

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kWavesM = 2;                  // wave grid of a workgroup
constexpr int kWavesN = 4;
constexpr int kWaves = kWavesM * kWavesN;
constexpr int kThreads = 64 * kWaves;
constexpr int kWM = kBM / kWavesM;          // wave tile rows
constexpr int kWN = kBN / kWavesN;          // wave tile cols
constexpr int kTM = kWM / 16;               // MFMA tiles per wave along M
constexpr int kTN = kWN / 16;               // MFMA tiles per wave along N
constexpr int kGA = kBM / 8 / kWaves;       // 8-row groups of A each wave loads per K step
constexpr int kGB = kBN / 8 / kWaves;       // ... and of B
constexpr int kGroupM = 8;         // tiles per raster group along M
// s_waitcnt immediate for vmcnt(0) alone (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8])
constexpr int kWaitVmcnt0 = 0x0F70;

struct Operand {
    const uint16_t *p;   // row-major [rows, K] bf16 bits
    int64_t ld;          // row stride in elements (multiple of 8)
    int rows;
};

// Workgroup -> output tile.  Workgroups are dispatched round-robin over the 8
// XCDs (bid % 8); remap so each XCD gets one contiguous range of tile ids,
// then walk that range in groups of kGroupM tiles along M so that the tiles
// running together on one XCD share A and B panels in its L2.
__device__ __forceinline__ void tile_of_block(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
    const int total = tiles_m * tiles_n;
    const int q = total >> 3, r = total & 7;
    const int xcd = bid & 7, local = bid >> 3;
    const int pid = xcd * q + min(xcd, r) + local;
    const int width = kGroupM * tiles_n;
    const int group = pid / width;
    const int first_m = group * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int in_group = pid - group * width;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

typedef f32x4 Acc[kTM][kTN];

typedef __attribute__((address_space(3))) void lds_void;

// dword 3 of a gfx9 raw buffer resource (32-bit data format; no swizzle, no index)
constexpr int kBufferFlags = 0x00020000;
// resources are capped at 1 GiB (no K step of a 256-row panel reaches further when
// its rows are shorter than 2M elements); this offset is past all of them
constexpr uint32_t kResourceCap = 1u << 30;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ uint32_t resource_bytes(int64_t b) {
    return b <= 0 ? 0u : (b >= (int64_t)kResourceCap ? kResourceCap : (uint32_t)b);
}

// A raw buffer resource over `bytes` bytes from `base` (capped as above).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, resource_bytes(bytes), kBufferFlags);
}

// 16-byte store through a buffer resource: the hardware drops a store whose offset
// lies outside the resource, so ragged tile edges need no branch.  kPolicy is the
// instruction's cache-policy field; kStoreNT (bit 1, "nt") marks the data
// non-temporal.  The backward's dlogits copies (2 x N x Vs bf16, far larger than L2)
// are stored that way so that they do not evict the operand panels the
// neighbouring tiles are still reading; measured on the 8B-class shard, nt on
// the fp32 gradient stores was slightly slower, so those use the default policy.
constexpr int kStoreNT = 2;
constexpr int kStoreDefault = 0;
template <int kPolicy>
__device__ __forceinline__ void store16(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kPolicy);
}

// One K step of operand fragments held by a wave: 8 A rows-blocks and 8 B col-blocks.
struct Frags {
    bf16x8 a[kTM];
    bf16x8 b[kTN];
};

// two LDS stages of one [256 x 64] A tile and one [256 x 64] B tile each (2 x 64 KiB)
constexpr int kStage = (kBM + kBN) * kBK;

// One output tile of C = A B^T: block `bid` of a tiles_m x tiles_n grid, computed by
// the workgroup's kThreads threads with `smem` (2 kStage elements) as its LDS.
template <class Epilogue>
__device__ __forceinline__ void gemm_nt_tile(const Operand &A, const Operand &B, int K,
                                             int tiles_m, int tiles_n, const Epilogue &epi,
                                             int bid, uint16_t *smem) {
    int tm, tn;
    tile_of_block(bid, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
    const int wm = wave % kWavesM, wn = wave / kWavesM;

    // Global -> LDS map (buffer loads straight into LDS, 16 bytes per lane).  One wave
    // instruction fills 8 rows x 128 B = 1 KiB of LDS in lane order: lane L lands on
    // row L/8, physical chunk L%8, so it fetches the logical chunk (L%8) ^ (row & 7).
    // Wave w fills 8-row groups w*kGA .. (w+1)*kGA-1 of A and w*kGB .. of B.
    // The buffer resource starts at the tile's first row and ends at the tensor's
    // end, so rows past M (or N) fall outside it and read as zeros.
    const int lrow = lane >> 3;
    const int lchunk = (lane & 7) ^ lrow;
    const char *a_panel = (const char *)(A.p + (int64_t)m0 * A.ld);
    const char *b_panel = (const char *)(B.p + (int64_t)n0 * B.ld);
    // bytes from the panel start to the end of the last row (past it: zeros)
    const uint32_t a_bytes = resource_bytes((int64_t)(A.rows - m0) * A.ld * 2);
    const uint32_t b_bytes = resource_bytes((int64_t)(B.rows - n0) * B.ld * 2);
    const uint32_t a_row8 = (uint32_t)(8 * A.ld * 2), b_row8 = (uint32_t)(8 * B.ld * 2);
    const uint32_t a_off0 = (uint32_t)(((wave * kGA * 8 + lrow) * A.ld + lchunk * 8) * 2);
    const uint32_t b_off0 = (uint32_t)(((wave * kGB * 8 + lrow) * B.ld + lchunk * 8) * 2);
    const int grp_a = wave * kGA * 8 * kBK;   // LDS element offsets of this wave's first groups
    const int grp_b = kBM * kBK + wave * kGB * 8 * kBK;

    // Branch-free: a chunk at or past K (the last partial K step, or a step past the
    // end) gets an offset outside the resource, which reads as zeros.
    auto load_tile = [&](uint16_t *buf, int k0) {
        const __amdgpu_buffer_rsrc_t ra =
            __builtin_amdgcn_make_buffer_rsrc((void *)(a_panel + 2 * k0), (short)0, a_bytes, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rb =
            __builtin_amdgcn_make_buffer_rsrc((void *)(b_panel + 2 * k0), (short)0, b_bytes, kBufferFlags);
        const bool ok = k0 + lchunk * 8 < K;
        const uint32_t oa = ok ? a_off0 : kOutOfRange;
        const uint32_t ob = ok ? b_off0 : kOutOfRange;
#pragma unroll
        for (int i = 0; i < kGA; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)(buf + grp_a + i * 8 * kBK), 16,
                                                     oa + i * a_row8, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < kGB; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(buf + grp_b + i * 8 * kBK), 16,
                                                     ob + i * b_row8, 0, 0, 0);
    };

    // fragment map: lane reads row (lane & 15) of each 16-row tile, logical chunk kk*4 + lane/16
    const int fr = lane & 15;
    const int a_off = (wm * kWM + fr) * kBK;
    const int b_off = kBM * kBK + (wn * kWN + fr) * kBK;
    const int ch0 = ((0 + (lane >> 4)) ^ (fr & 7)) * 8;
    const int ch1 = ((4 + (lane >> 4)) ^ (fr & 7)) * 8;

    auto read_frags = [&](const uint16_t *buf, int ch, Frags &f) {
#pragma unroll
        for (int i = 0; i < kTM; ++i) f.a[i] = *(const bf16x8 *)&buf[a_off + i * 16 * kBK + ch];
#pragma unroll
        for (int j = 0; j < kTN; ++j) f.b[j] = *(const bf16x8 *)&buf[b_off + j * 16 * kBK + ch];
    };

    Acc acc;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto mma = [&](const Frags &f, int i0, int i1) {
#pragma unroll
        for (int i = i0; i < i1; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
    };

    const int KT = (int)ceil_div(K, kBK);
    constexpr int kReads = kTM + kTN;    // LDS fragment reads per half K step
    constexpr int kMfmas = kTM * kTN;    // MFMAs per half K step
    static_assert(kMfmas >= 2 * kReads && kMfmas >= kGA + kGB + kReads, "schedule shape");
    Frags f0, f1;

    load_tile(smem, 0);
    load_tile(smem + kStage, kBK);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    read_frags(smem, ch0, f0);

    // K step kt works on the tile in stage kt & 1; the next tile is in the other stage.
    // F0 (K 0..31 of the step) is already in registers when the step starts.  The
    // sched_group_barrier masks: 0x008 MFMA, 0x100 LDS read, 0x020 global/buffer load.
    for (int kt = 0; kt < KT; ++kt) {
        uint16_t *cur = smem + (kt & 1) * kStage;
        uint16_t *nxt = smem + ((kt + 1) & 1) * kStage;
        // phase 1: F0's MFMAs, with F1's LDS reads spread over the first of them
        read_frags(cur, ch1, f1);
        mma(f0, 0, kTM);
#pragma unroll
        for (int q = 0; q < kReads; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kMfmas - 2 * kReads, 0);
        __builtin_amdgcn_sched_barrier(0);
        // every wave has its F1 (nobody reads `cur` any more) and tile kt+1 has landed;
        // no branch: past the last step the loads read zeros and F0 is unused
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        // phase 2: F1's MFMAs, with tile kt+2's loads and the next F0's reads
        load_tile(cur, (kt + 2) * kBK);
        read_frags(nxt, ch0, f0);
        mma(f1, 0, kTM);
#pragma unroll
        for (int q = 0; q < kGA + kGB; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
#pragma unroll
        for (int q = 0; q < kReads; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kMfmas - kGA - kGB - kReads, 0);
        __builtin_amdgcn_sched_barrier(0);
    }

    // The last steps' loads (zeros) may still be landing and other waves may still be
    // reading: drain both before an epilogue reuses the LDS.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();

    // accumulator layout of v_mfma_f32_16x16x32: acc[i][j][r] is
    //   row m0 + wm*kWM + 16 i + 4 (lane / 16) + r,  column n0 + wn*kWN + 16 j + (lane % 16)
    // The epilogue may use the 128 KiB of LDS (`smem`); all kThreads threads call it.
    epi(acc, m0 + wm * kWM, n0 + wn * kWN, lane, m0, n0, smem);
}

template <class Epilogue>
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_kernel(Operand A, Operand B, int K,
                                                              int tiles_m, int tiles_n,
                                                              Epilogue epi) {
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * kStage];
    gemm_nt_tile(A, B, K, tiles_m, tiles_n, epi, blockIdx.x, smem);
}

// out[n, m] = C[m, n] (fp32), m < M, n < N.  Stores are 4 rows of C (16 bytes) at a time:
// when M is not a multiple of 4, the last chunk also writes C's zero rows past M into the
// row's padding, so ldo must be a multiple of 4 (>= M).  Stores go through a
// resource over the output rows from the workgroup's first one: rows past N are
// outside it, columns past M get an offset outside it.
struct StoreTransposedEpilogue {
    float *out;
    int64_t ldo;
    int M, N;

    __device__ __forceinline__ void operator()(Acc &acc, int mbase, int nbase, int lane, int m0,
                                               int n0, uint16_t *) const {
        const int rsub = 4 * (lane >> 4);
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(out + (int64_t)n0 * ldo + m0, ((int64_t)(N - n0) * ldo - m0) * 4);
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int64_t nl = nbase - n0 + 16 * j + (lane & 15);
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const int ml = mbase - m0 + 16 * i + rsub;
                store16<kStoreDefault>(__builtin_bit_cast(u32x4, acc[i][j]), rs,
                        m0 + ml < M ? (uint32_t)((nl * ldo + ml) * 4) : kOutOfRange);
            }
        }
    }
};

// Launch geometry of a GEMM over an M x N output.
struct GemmGrid {
    int tiles_m, tiles_n;
    int blocks() const { return tiles_m * tiles_n; }
};
inline GemmGrid gemm_grid(int64_t M, int64_t N) {
    return GemmGrid{(int)ceil_div(M, kBM), (int)ceil_div(N, kBN)};
}

}  // namespace vp
