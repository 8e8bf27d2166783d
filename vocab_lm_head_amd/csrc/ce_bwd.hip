// Local backward of one vocabulary shard.
//
// Method: MiniMind-Tron "5 Vocab Parallelism", 5.3.2 -- dCE/dz_j = p_j - [j == y],
// with p from the local logits and the global log-sum-exp, and the one-hot
// subtracted only on the shard that owns the target; no communication.  5.3.3:
// ignored tokens get zero gradient and the mean divides by max(1, N_valid).
// The input gradient of this shard is a partial sum (column-parallel linear,
// glossary "Tensor Parallelism"); the weight gradient is local.
//
// Steps (all on the caller's stream):
//   1. X -> X^T and W_r -> W_r^T (bf16, rows zero-padded to a multiple of 64
//      elements), so that all three GEMMs are K-contiguous on both operands;
//   2. recompute z^T = W_r X^T on MFMA; the epilogue forms
//      dz = g (exp(z - lse) - onehot) in registers, stages the tile in LDS and
//      writes it in bf16 twice, token-major dz [N, Vs64] and vocab-major dz^T [Vs, N64];
//   3. dX_r^T = W_r^T dz^T  (A = W_r^T [H, Vs64], B = dz [N, Vs64]), K = Vs64
//   4. dW_r^T = X^T dz      (A = X^T [H, N64],   B = dz^T [Vs, N64]),  K = N64
// The [N, Vs] dlogits must reach memory once: a register-only fusion of dX and
// dW would need fp32 atomics on [tile, H] slabs for every tile, far below the
// MFMA roofline at H = 4096.
#include <algorithm>

#include "gemm.hpp"
#include "launch.hpp"

namespace vp {

namespace {

// out[c, r] = in[r, c] for r < rows, c < cols; out[c, r] = 0 for rows <= r < ld_out.
// in: [rows, cols] row-major (cols multiple of 8); out: [cols, ld_out] (ld_out multiple of 8).
constexpr int kTT = 64;
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t *__restrict__ in,
                                                             int64_t rows, int64_t cols,
                                                             uint16_t *__restrict__ out,
                                                             int64_t ld_out) {
    __shared__ uint16_t tile[kTT][kTT + 2];
    const int64_t r0 = (int64_t)blockIdx.x * kTT;   // input rows  = output columns
    const int64_t c0 = (int64_t)blockIdx.y * kTT;   // input cols  = output rows
    const int t = threadIdx.x;
    {
        const int r = t >> 2, cc = (t & 3) * 16;
        const int64_t gr = r0 + r;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t gc = c0 + cc + 8 * half;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (gr < rows && gc < cols) v = *(const u32x4 *)(in + gr * cols + gc);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                tile[r][cc + 8 * half + 2 * q] = (uint16_t)(v[q] & 0xFFFFu);
                tile[r][cc + 8 * half + 2 * q + 1] = (uint16_t)(v[q] >> 16);
            }
        }
    }
    __syncthreads();
    {
        const int oc = t >> 2, rr = (t & 3) * 16;   // output row c0 + oc, output cols r0 + rr ..
        const int64_t grow = c0 + oc;
        if (grow >= cols) return;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int64_t gcol = r0 + rr + 8 * half;
            if (gcol >= ld_out) continue;
            u32x4 v;   // rows past `rows` were staged as zeros
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v[q] = (unsigned)tile[rr + 8 * half + 2 * q][oc] |
                       ((unsigned)tile[rr + 8 * half + 2 * q + 1][oc] << 16);
            *(u32x4 *)(out + grow * ld_out + gcol) = v;
        }
    }
}

hipError_t transpose_bf16(const uint16_t *in, int64_t rows, int64_t cols, uint16_t *out,
                          int64_t ld_out, hipStream_t stream) {
    dim3 grid((unsigned)ceil_div(ld_out, kTT), (unsigned)ceil_div(cols, kTT));
    hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, stream, in, rows, cols, out, ld_out);
    return hipGetLastError();
}

// dz = g (softmax - onehot) from the recomputed z^T tile; rows = vocab, cols = tokens.
// The 256 x 256 bf16 tile is staged in the GEMM's LDS as [token][vocab] rows of
// 512 bytes, then written out with 16-byte coalesced stores twice: token-major
// dz [N, ld_dz] and vocab-major dz^T [M, ld_dzt].  Padding columns (vocab >= M,
// token >= N) are written as zeros.
static_assert(kBN * kBM <= 2 * (kBM + kBN) * kBK, "dz tile must fit the GEMM's LDS");

// Element offset of (row, col) in the staged tile: 16-byte chunks are XOR-swizzled
// with (row ^ row/8) so that 16 consecutive rows at one column (the MFMA-layout
// writes) and rows 8 apart at one column (the vocab-major reads) fall in
// different banks, while a row read stays one contiguous permuted row.
__device__ __forceinline__ int dz_swz(int row, int col) {
    return row * kBM + ((((col >> 3) ^ ((row ^ (row >> 3)) & 31)) << 3) | (col & 7));
}

struct DlogitsEpilogue {
    const int64_t *targets;
    const float *lse;
    int64_t start;
    int64_t ignore_index;
    float grad_scale;
    int M, N;              // Vs, tokens
    int64_t ld_dz, ld_dzt; // padded leading dims (multiples of 64)
    uint16_t *dz;          // [N, ld_dz]
    uint16_t *dzt;         // [M, ld_dzt]

    __device__ __forceinline__ void operator()(Acc &acc, int mbase, int nbase, int lane, int m0,
                                               int n0, uint16_t *lds) const {
        const int rsub = 4 * (lane >> 4);
        // the lane's targets and lse values, all loaded before any is used (one memory
        // latency per tile); columns past N read token N-1 and are masked below
        int64_t tg[kTN];
        float ls[kTN];
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int nc = min(nbase + 16 * j + (lane & 15), N - 1);
            tg[j] = targets[nc];
            ls[j] = lse[nc];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int n = nbase + 16 * j + (lane & 15);
            const bool ncol = n < N;
            const float g = (tg[j] == ignore_index) ? 0.f : grad_scale;
            const float lsel = ls[j] * kLog2e;
            const int64_t trow = tg[j] - start;
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                const int row0 = mbase + 16 * i + rsub;   // vocabulary row of r = 0
                float d[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = fast_exp2(fmaf(acc[i][j][r], kLog2e, -lsel));
                    const float v = g * (p - ((row0 + r) == trow ? 1.f : 0.f));
                    d[r] = (ncol && (row0 + r) < M) ? v : 0.f;   // padding stays exactly 0
                }
                *(u32x2 *)(lds + dz_swz(n - n0, row0 - m0)) = pack_bf16x4(d[0], d[1], d[2], d[3]);
            }
        }
        __syncthreads();
        const int t = threadIdx.x;
        // Both passes read all of their LDS chunks first, then issue their stores; rows
        // past N (or M) lie outside the store resource and are dropped by the hardware,
        // padding columns past the leading dimension get an offset outside it.
        {   // token-major: thread t owns 16-byte chunk t % 32 of rows t/32 + 16 it
            const int c = t & 31, r0 = t >> 5;
            constexpr int kIt = (kBN * kBM / 8) / kThreads;
            constexpr int kRowStep = kThreads / 32;
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(dz + (int64_t)n0 * ld_dz + m0, ((int64_t)(N - n0) * ld_dz - m0) * 2);
            const bool colok = m0 + 8 * c < ld_dz;
            u32x4 v[kIt];
#pragma unroll
            for (int it = 0; it < kIt; ++it)
                v[it] = *(const u32x4 *)(lds + dz_swz(r0 + kRowStep * it, 8 * c));
#pragma unroll
            for (int it = 0; it < kIt; ++it)
                store16<kStoreNT>(v[it], rs,
                        colok ? (uint32_t)(((int64_t)(r0 + kRowStep * it) * ld_dz + 8 * c) * 2) : kOutOfRange);
        }
        {   // vocab-major: a lane gathers 4 vocab rows x 8 tokens (eight 8-byte LDS reads)
            // per iteration and writes four 16-byte chunks; 32 lanes cover a 512-byte row
            const int c = (t & 31) * 8, vq = (t >> 5) * 4;
            constexpr int kIt = (kBM * kBN / 32) / kThreads;
            constexpr int kVocabStep = 4 * kThreads / 32;
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(dzt + (int64_t)m0 * ld_dzt + n0, ((int64_t)(M - m0) * ld_dzt - n0) * 2);
            const bool colok = n0 + c < ld_dzt;
            u32x2 rd[kIt][8];
#pragma unroll
            for (int it = 0; it < kIt; ++it)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    rd[it][e] = *(const u32x2 *)(lds + dz_swz(c + e, vq + kVocabStep * it));
#pragma unroll
            for (int it = 0; it < kIt; ++it)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int w = v >> 1, sh = (v & 1) * 16;
                    u32x4 o;
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        o[p] = ((rd[it][2 * p][w] >> sh) & 0xFFFFu) |
                               (((rd[it][2 * p + 1][w] >> sh) & 0xFFFFu) << 16);
                    const int64_t row = vq + kVocabStep * it + v;
                    store16<kStoreNT>(o, rs, colok ? (uint32_t)((row * ld_dzt + c) * 2) : kOutOfRange);
                }
        }
    }
};

__global__ void fill_zero_kernel(float *p, int64_t count) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

// Split-K form of the transposed store: the grid holds `splits` copies of the tile grid,
// and copy s computes every tile over the K columns [s chunk, min((s + 1) chunk, K)) of
// both operands (chunk a multiple of kBK, so the shifted rows stay 128-byte aligned) and
// stores its partial at epi.out + s out_stride.  A reduction then sums the partials in
// split order.  For outputs with too few tiles to fill the chip.
__global__ __launch_bounds__(kThreads, 1) void gemm_nt_splitk_store_kernel(
    Operand A, Operand B, int K, int chunk, int tiles_m, int tiles_n, StoreTransposedEpilogue epi,
    int64_t out_stride) {
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * kStage];
    const int tiles = tiles_m * tiles_n;
    const int split = blockIdx.x / tiles;
    const int k0 = split * chunk;
    Operand a = A, b = B;
    a.p += k0;
    b.p += k0;
    epi.out += split * out_stride;
    gemm_nt_tile(a, b, min(chunk, K - k0), tiles_m, tiles_n, epi, blockIdx.x - split * tiles, smem);
}

// out[i] = sum over s of part[s stride + i] for i < count, in split order (fp32).  count
// and stride are multiples of 4 and the buffers 16-byte aligned.
constexpr int kMaxSplits = 16;
__global__ __launch_bounds__(256) void sum_splits_kernel(const float *__restrict__ part, int splits,
                                                         int64_t count, int64_t stride,
                                                         float *__restrict__ out) {
    const f32x4 *p = (const f32x4 *)part;
    const int64_t n4 = count / 4, s4 = stride / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * blockDim.x) {
        f32x4 v[kMaxSplits];
#pragma unroll
        for (int s = 0; s < kMaxSplits; ++s)
            if (s < splits) v[s] = p[s * s4 + i];
        f32x4 acc = v[0];
#pragma unroll
        for (int s = 1; s < kMaxSplits; ++s)
            if (s < splits) acc += v[s];
        ((f32x4 *)out)[i] = acc;
    }
}

// K splits of a gradient GEMM with `tiles` output tiles: below one tile per CU the K
// loop is split (aiming at kSplitTargetBlocks workgroups, at least kSplitMinSteps K
// steps each); chunk is a multiple of kBK.
constexpr int64_t kSplitMinTiles = 256;
constexpr int64_t kSplitTargetBlocks = 512;
constexpr int64_t kSplitMinSteps = 8;
void grad_split(int64_t tiles, int64_t K, int64_t &splits, int64_t &chunk) {
    splits = 1;
    if (tiles < kSplitMinTiles)
        splits = std::max<int64_t>(1, std::min({ceil_div(kSplitTargetBlocks, tiles),
                                                K / (kBK * kSplitMinSteps), (int64_t)kMaxSplits}));
    chunk = round_up(ceil_div(K, splits), kBK);
    splits = ceil_div(K, chunk);
}

}  // namespace

BwdWorkspace bwd_workspace(int64_t n, int64_t h, int64_t vs) {
    BwdWorkspace b;
    // leading dimensions padded to 64 elements: every workspace row starts on a
    // 128-byte line, so a 64-element K chunk of a GEMM operand is one line
    b.n_ld = round_up(n, 64);
    b.vs_ld = round_up(vs, 64);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (size_t)round_up((int64_t)bytes, 256);
        return o;
    };
    b.off_xt = take((size_t)h * b.n_ld * 2);
    b.off_wt = take((size_t)h * b.vs_ld * 2);
    b.off_dz = take((size_t)n * b.vs_ld * 2);
    b.off_dzt = take((size_t)vs * b.n_ld * 2);
    grad_split(gemm_grid(h, n).blocks(), b.vs_ld, b.splits_dx, b.chunk_dx);
    grad_split(gemm_grid(h, vs).blocks(), b.n_ld, b.splits_dw, b.chunk_dw);
    const int64_t part = std::max(b.splits_dx > 1 ? b.splits_dx * n * h : 0,
                                  b.splits_dw > 1 ? b.splits_dw * vs * h : 0);
    b.off_split = take((size_t)part * 4);
    b.bytes = off;
    return b;
}

hipError_t launch_bwd_transposes(const uint16_t *x, const uint16_t *w, int64_t n, int64_t h,
                                 int64_t vs, void *ws, hipStream_t stream) {
    const BwdWorkspace b = bwd_workspace(n, h, vs);
    char *base = (char *)ws;
    hipError_t e;
    if ((e = transpose_bf16(x, n, h, (uint16_t *)(base + b.off_xt), b.n_ld, stream)) != hipSuccess)
        return e;
    return transpose_bf16(w, vs, h, (uint16_t *)(base + b.off_wt), b.vs_ld, stream);
}

hipError_t launch_bwd_grad_gemms(int64_t n, int64_t h, int64_t vs, float *dx, float *dw, void *ws,
                                 hipStream_t stream) {
    const BwdWorkspace b = bwd_workspace(n, h, vs);
    char *base = (char *)ws;
    const uint16_t *xt = (const uint16_t *)(base + b.off_xt);
    const uint16_t *wt = (const uint16_t *)(base + b.off_wt);
    const uint16_t *dz = (const uint16_t *)(base + b.off_dz);
    const uint16_t *dzt = (const uint16_t *)(base + b.off_dzt);
    float *part = (float *)(base + b.off_split);
    // C^T [H, cols] = A [H, K] . B [cols, K]^T stored as out [cols, H]; split over K (into
    // the partials, then summed into out) when the output has too few tiles
    auto gemm = [&](Operand A, Operand B, int64_t K, int64_t cols, int64_t splits, int64_t chunk,
                    float *out) -> hipError_t {
        const GemmGrid g = gemm_grid(h, cols);
        if (splits == 1) {
            StoreTransposedEpilogue epi{out, h, (int)h, (int)cols};
            hipLaunchKernelGGL(gemm_nt_kernel<StoreTransposedEpilogue>, dim3(g.blocks()),
                               dim3(kThreads), 0, stream, A, B, (int)K, g.tiles_m, g.tiles_n, epi);
            return hipGetLastError();
        }
        StoreTransposedEpilogue epi{part, h, (int)h, (int)cols};
        hipLaunchKernelGGL(gemm_nt_splitk_store_kernel, dim3((unsigned)(g.blocks() * splits)),
                           dim3(kThreads), 0, stream, A, B, (int)K, (int)chunk, g.tiles_m,
                           g.tiles_n, epi, cols * h);
        const int64_t count = cols * h;
        hipLaunchKernelGGL(sum_splits_kernel,
                           dim3((unsigned)std::min<int64_t>(ceil_div(count / 4, 256), 8192)),
                           dim3(256), 0, stream, part, (int)splits, count, count, out);
        return hipGetLastError();
    };
    hipError_t e;
    // dX_r^T [H, N] = W_r^T [H, Vs64] . dz [N, Vs64]^T
    if ((e = gemm(Operand{wt, b.vs_ld, (int)h}, Operand{dz, b.vs_ld, (int)n}, b.vs_ld, n,
                  b.splits_dx, b.chunk_dx, dx)) != hipSuccess)
        return e;
    // dW_r^T [H, Vs] = X^T [H, N64] . dz^T [Vs, N64]^T
    return gemm(Operand{xt, b.n_ld, (int)h}, Operand{dzt, b.n_ld, (int)vs}, b.n_ld, vs, b.splits_dw,
                b.chunk_dw, dw);
}

hipError_t launch_bwd_zero_dw(float *dw, int64_t vs, int64_t h, hipStream_t stream) {
    const int64_t cnt = vs * h;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)std::min<int64_t>(ceil_div(cnt, 256), 8192)),
                       dim3(256), 0, stream, dw, cnt);
    return hipGetLastError();
}

hipError_t launch_ce_bwd(const uint16_t *x, const uint16_t *w, const int64_t *targets,
                         const float *lse, int64_t n, int64_t h, int64_t start, int64_t vs,
                         int64_t ignore_index, float grad_scale, float *dx, float *dw, void *ws,
                         hipStream_t stream) {
    if (n == 0) return launch_bwd_zero_dw(dw, vs, h, stream);   // no tokens: dW is zero
    const BwdWorkspace b = bwd_workspace(n, h, vs);
    char *base = (char *)ws;
    uint16_t *dz = (uint16_t *)(base + b.off_dz);
    uint16_t *dzt = (uint16_t *)(base + b.off_dzt);
    hipError_t e;
    if ((e = launch_bwd_transposes(x, w, n, h, vs, ws, stream)) != hipSuccess) return e;
    {   // recompute + dlogits: rows = vocab (A = W_r), cols = tokens (B = X)
        const GemmGrid g = gemm_grid(vs, n);
        DlogitsEpilogue epi{targets, lse, start, ignore_index, grad_scale, (int)vs, (int)n,
                            b.vs_ld, b.n_ld, dz, dzt};
        hipLaunchKernelGGL(gemm_nt_kernel<DlogitsEpilogue>, dim3(g.blocks()), dim3(kThreads), 0,
                           stream, Operand{w, h, (int)vs}, Operand{x, h, (int)n}, (int)h,
                           g.tiles_m, g.tiles_n, epi);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_bwd_grad_gemms(n, h, vs, dx, dw, ws, stream);
}

}  // namespace vp
