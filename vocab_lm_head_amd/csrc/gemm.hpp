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
// Global -> LDS goes through buffer loads straight into LDS (buffer_load ... lds).
//
// Ping-pong schedule.  The CU places wave w and wave w + 4 of a workgroup on the same
// SIMD (measured with the HW_ID register), so waves 0-3 (group 0) and 4-7 (group 1)
// each hold one wave per SIMD.  The groups run half a K step apart, separated by
// workgroup barriers: in each interval one group reads a whole K step's fragments
// from LDS and issues its global loads while the other runs that step's 64 MFMAs, so
// the SIMD's matrix core is fed by one wave while the other waits on memory.  Group g
// computes M half g; group 0 loads the A tiles, group 1 the B tiles.  With K step k in
// LDS stage k % 2, interval 2k holds group 0's reads of step k and its loads of A(k+1)
// (into the other stage, which group 1 finished reading in interval 2k - 1); interval
// 2k + 1 holds group 1's reads of step k, then, once they are complete, its loads of
// B(k+2) into the same stage (group 0 read it in interval 2k).  Each load has landed
// before the interval of its first read begins.  That early B load relies on each wave of
// group 1 reading exactly the 64 B rows it loads itself (its N columns are its slab): the
// wave's own wait for its reads is then the only one needed before it overwrites them.
// A layout in which one wave reads rows another wave of its group loads would need a
// barrier there instead.
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

// One K step of operand fragments held by a wave: for each 32-wide half of the step,
// kTM A row blocks and kTN B column blocks.
struct Frags {
    bf16x8 a[2][kTM];
    bf16x8 b[2][kTN];
};

static_assert(kWaves == 8 && kWavesM == 2 && kBM == kBN && kBM / kWavesN == 64,
              "ping-pong layout: two groups of four waves, one 64-row load slab per wave");
// load instructions one wave issues per K step: its 64-row slab, 8 rows per instruction
constexpr int kSlabLoads = kBM / kWavesN / 8;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8])
constexpr int wait_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kWaitLgkmcnt0 = 0xC07F;

// A workgroup barrier that orders nothing by itself: the memory waits around it are
// explicit, so that loads may stay in flight across it.  The empty asm statements keep
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

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
    const int grp = wave >> 2, slab = wave & 3;   // group; the wave's place in it (its SIMD)
    const int wm = grp, wn = slab;   // wn == slab: a wave reads the B rows it loads

    // Global -> LDS map (buffer loads straight into LDS, 16 bytes per lane).  One wave
    // instruction fills 8 rows x 128 B = 1 KiB of LDS in lane order: lane L lands on
    // row L/8, physical chunk L%8, so it fetches the logical chunk (L%8) ^ (row & 7).
    // Group 0 loads A and group 1 loads B; wave `slab` of a group loads rows
    // 64 slab .. 64 slab + 63 of its operand's tile, eight instructions per K step.
    // The buffer resource starts at the tile's first row and ends at the tensor's
    // end, so rows past M (or N) fall outside it and read as zeros.
    const Operand &L = grp ? B : A;
    const int r0 = grp ? n0 : m0;
    const int lrow = lane >> 3;
    const int lchunk = (lane & 7) ^ lrow;
    const char *panel = (const char *)(L.p + (int64_t)r0 * L.ld);
    // bytes from the panel start to the end of the last row (past it: zeros)
    const uint32_t bytes = resource_bytes((int64_t)(L.rows - r0) * L.ld * 2);
    const uint32_t row8 = (uint32_t)(8 * L.ld * 2);
    const uint32_t off0 = (uint32_t)(((64 * slab + lrow) * L.ld + lchunk * 8) * 2);
    const int dst0 = (grp ? kBM * kBK : 0) + 64 * slab * kBK;   // LDS element offset in a stage

    // Branch-free: a chunk at or past K (the last partial K step, or a step past the
    // end) gets an offset outside the resource, which reads as zeros.
    auto load_slab = [&](int st, int k0) {
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc((void *)(panel + 2 * k0), (short)0, bytes, kBufferFlags);
        const uint32_t o = k0 + lchunk * 8 < K ? off0 : kOutOfRange;
        uint16_t *dst = smem + st * kStage + dst0;
#pragma unroll
        for (int i = 0; i < kSlabLoads; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + i * 8 * kBK), 16,
                                                     o + i * row8, 0, 0, 0);
    };

    // fragment map: lane reads row (lane & 15) of each 16-row tile, logical chunk kk*4 + lane/16
    const int fr = lane & 15;
    const int a_off = (wm * kWM + fr) * kBK;
    const int b_off = kBM * kBK + (wn * kWN + fr) * kBK;
    const int ch[2] = {((0 + (lane >> 4)) ^ (fr & 7)) * 8, ((4 + (lane >> 4)) ^ (fr & 7)) * 8};

    auto read_step = [&](int st, Frags &f) {
        const uint16_t *buf = smem + st * kStage;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int i = 0; i < kTM; ++i) f.a[kk][i] = *(const bf16x8 *)&buf[a_off + i * 16 * kBK + ch[kk]];
#pragma unroll
            for (int j = 0; j < kTN; ++j) f.b[kk][j] = *(const bf16x8 *)&buf[b_off + j * 16 * kBK + ch[kk]];
        }
    };

    Acc acc;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto mma_step = [&](const Frags &f) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[kk][i], f.b[kk][j], acc[i][j], 0, 0, 0);
    };

    const int KT = (int)ceil_div(K, kBK);
    // Prologue: A(0) from group 0, B(0) and B(1) from group 1.  Group 1 then sits out
    // interval 0 and group 0 the last interval, so every wave passes 2 KT + 3 barriers
    // (this one, the two per K step, the extra one and the one before the epilogue).
    load_slab(0, 0);
    if (grp == 0) {
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    } else {
        load_slab(1, kBK);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(kSlabLoads));   // B(0) has landed; B(1) may be in flight
    }
    bare_barrier();
    if (grp == 1) bare_barrier();
    Frags f;
    for (int k = 0; k < KT; ++k) {
        const int st = k & 1;
        // memory interval: this K step's fragments, then the group's loads
        read_step(st, f);
        if (grp == 0) {
            load_slab(st ^ 1, (k + 1) * kBK);              // A(k+1)
        } else {
            __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);     // this wave's reads of stage st are done
            load_slab(st, (k + 2) * kBK);                  // B(k+2)
            __builtin_amdgcn_s_waitcnt(wait_vmcnt(kSlabLoads));   // B(k+1) has landed
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
        bare_barrier();
        // compute interval: the step's 64 MFMAs
        mma_step(f);
        __builtin_amdgcn_sched_barrier(0);
        if (grp == 0) __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));   // A(k+1) has landed
        bare_barrier();
    }
    if (grp == 0) bare_barrier();

    // Past the last K step the loads (zeros) may still be landing: drain them before an
    // epilogue reuses the LDS.
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
