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
// Tiling (one workgroup = 4 waves of 64 lanes, one workgroup per CU):
//   block tile 256 (M) x 256 (N), K step 64, LDS double buffer 2 x 64 KiB;
//   wave (wm, wn) owns a 128 x 128 sub-tile = 8 x 8 MFMA tiles of
//   v_mfma_f32_16x16x32_bf16 with fp32 accumulators (256 per lane).
// LDS rows are 64 bf16 = 128 B = eight 16-byte chunks; chunk c of row r is
// stored at chunk c ^ (r & 7) so that the 16-lane groups of a fragment read
// (16 consecutive rows, one chunk) hit distinct banks.
// Global -> LDS staging goes through registers: the loads of step k+1 are
// issued before the MFMAs of step k and written to the other LDS buffer
// after them, with one barrier per K step.
//
// Rows past M / N are clamped to the last row (their results are masked by
// the epilogue); K chunks past K are zero-filled, so K need only be a multiple
// of 8.  Operands must have 16-byte aligned rows.
#pragma once

#include "common.hpp"

namespace vp {

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kThreads = 256;
constexpr int kWM = 128;           // wave tile rows
constexpr int kWN = 128;           // wave tile cols
constexpr int kTM = kWM / 16;      // MFMA tiles per wave along M
constexpr int kTN = kWN / 16;      // MFMA tiles per wave along N
constexpr int kGroupM = 8;         // tiles per raster group along M

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

template <class Epilogue>
__global__ __launch_bounds__(kThreads) void gemm_nt_kernel(Operand A, Operand B, int K,
                                                           int tiles_m, int tiles_n, Epilogue epi) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[2][(kBM + kBN) * kBK];

    int tm, tn;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * kBM, n0 = tn * kBN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    // staging map: 16-byte chunk c of rows rs + 32 i, i = 0..7, for A and for B
    const int c = tid & 7, rs = tid >> 3;
    const int kc = c * 8;
    const int st_off = rs * kBK + ((c ^ (rs & 7)) * 8);   // LDS element offset of row rs
    const uint16_t *a_row[8];
    const uint16_t *b_row[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int ra = min(m0 + rs + 32 * i, A.rows - 1);
        const int rb = min(n0 + rs + 32 * i, B.rows - 1);
        a_row[i] = A.p + (int64_t)ra * A.ld + kc;
        b_row[i] = B.p + (int64_t)rb * B.ld + kc;
    }

    // fragment map: lane reads row (lane & 15) of each 16-row tile, logical chunk kk*4 + lane/16
    const int fr = lane & 15;
    int frag_off[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) frag_off[kk] = fr * kBK + (((kk * 4 + (lane >> 4)) ^ (fr & 7)) * 8);
    const int a_base = (wm * kWM) * kBK;
    const int b_base = kBM * kBK + (wn * kWN) * kBK;

    Acc acc;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 sa[8], sb[8];
    auto gload = [&](int k0) {
        const bool ok = (k0 + kc) < K;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sa[i] = ok ? *(const u32x4 *)(a_row[i] + k0) : u32x4{0u, 0u, 0u, 0u};
            sb[i] = ok ? *(const u32x4 *)(b_row[i] + k0) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            *(u32x4 *)&smem[buf][st_off + 32 * i * kBK] = sa[i];
            *(u32x4 *)&smem[buf][kBM * kBK + st_off + 32 * i * kBK] = sb[i];
        }
    };

    const int KT = (int)ceil_div(K, kBK);
    gload(0);
    lstore(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) gload((kt + 1) * kBK);
        const uint16_t *S = smem[cur];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            bf16x8 af[kTM], bfr[kTN];
#pragma unroll
            for (int i = 0; i < kTM; ++i) af[i] = *(const bf16x8 *)&S[a_base + i * 16 * kBK + frag_off[kk]];
#pragma unroll
            for (int j = 0; j < kTN; ++j) bfr[j] = *(const bf16x8 *)&S[b_base + j * 16 * kBK + frag_off[kk]];
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int j = 0; j < kTN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (more) lstore(cur ^ 1);
        __syncthreads();
    }

    // accumulator layout of v_mfma_f32_16x16x32: acc[i][j][r] is
    //   row m0 + wm*128 + 16 i + 4 (lane / 16) + r,  column n0 + wn*128 + 16 j + (lane % 16)
    epi(acc, m0 + wm * kWM, n0 + wn * kWN, lane);
}

// Launch geometry of a GEMM over an M x N output.
struct GemmGrid {
    int tiles_m, tiles_n;
    int blocks() const { return tiles_m * tiles_n; }
};
inline GemmGrid gemm_grid(int64_t M, int64_t N) {
    return GemmGrid{(int)ceil_div(M, kBM), (int)ceil_div(N, kBN)};
}

}  // namespace vp
