// Materialised-logits comparator: the same step with one shard's fp32 logits stored in
// HBM, as the pages' tensor-parallel baseline holds them ([S, B, V/T] per rank, in fp32).
// It exists beside the fused path to measure what that path saves; it is not the hot path.
//
// Method: MiniMind-Tron "5 Vocab Parallelism", 5.3.1 -- the statistics are taken in the
// pages' order when asked (first every shard's maximum, the all-reduce MAX, then each
// shard's sum of exponentials about the global maximum), or in one read about the
// shard's own maximum; 5.3.2 -- the backward forms p - onehot from the stored logits
// (no recompute) before the same dX and dW GEMMs as the fused path.
#include "gemm.hpp"
#include "launch.hpp"

namespace vp {

namespace {

// Per-token statistics of one shard's stored logits, one workgroup per token row.
// Without a reference maximum: (max, sum of exp about it, target logit), in one read;
// with one: (m_ref, sum of exp about m_ref, target logit).  Columns past Vs are skipped.
constexpr int kStatThreads = 256;
template <bool kRef>
__global__ __launch_bounds__(kStatThreads) void logits_stats_kernel(
    const float *__restrict__ logits, int64_t ld, const int64_t *__restrict__ targets,
    int64_t start, int64_t vs, const float *__restrict__ m_ref, float *__restrict__ m_out,
    float *__restrict__ s_out, float *__restrict__ zy_out) {
    __shared__ float sm[kStatThreads], ss[kStatThreads], sz[kStatThreads];
    const int t = threadIdx.x;
    const int64_t i = blockIdx.x;
    const float *row = logits + i * ld;
    const int64_t local = targets[i] - start;
    const float ref = kRef ? m_ref[i] : 0.f;
    float m = kRef ? ref : -INFINITY, s = 0.f, zy = 0.f;
    for (int64_t c = 4 * t; c < vs; c += 4 * kStatThreads) {
        const f32x4 v = *(const f32x4 *)(row + c);   // ld >= round_up(Vs, 4): in the row
        float z[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            z[k] = c + k < vs ? v[k] : -INFINITY;
            if (c + k == local && c + k < vs) zy = v[k];
        }
        if (!kRef) {
            const float m4 = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
            if (m4 > m) {
                s *= fast_exp2((m - m4) * kLog2e);
                m = m4;
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) s += fast_exp2((z[k] - m) * kLog2e);
    }
    sm[t] = m;
    ss[t] = s;
    sz[t] = zy;
    __syncthreads();
    for (int w = kStatThreads / 2; w > 0; w >>= 1) {
        if (t < w) {
            if (kRef) {
                ss[t] += ss[t + w];
            } else {
                const float a = sm[t], b = sm[t + w], mx = fmaxf(a, b);
                const float sa = ss[t] != 0.f ? ss[t] * fast_exp2((a - mx) * kLog2e) : 0.f;
                const float sb = ss[t + w] != 0.f ? ss[t + w] * fast_exp2((b - mx) * kLog2e) : 0.f;
                sm[t] = mx;
                ss[t] = sa + sb;
            }
            sz[t] += sz[t + w];
        }
        __syncthreads();
    }
    if (t == 0) {
        m_out[i] = kRef ? ref : sm[0];
        s_out[i] = ss[0];
        zy_out[i] = sz[0];
    }
}

// m_max[i] = max over the T rows of m [T, n]: the all-reduce MAX on one GPU.
__global__ __launch_bounds__(256) void rows_max_kernel(const float *__restrict__ m, int64_t n,
                                                       int T, float *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float v = -INFINITY;
    for (int r = 0; r < T; ++r) v = fmaxf(v, m[(int64_t)r * n + i]);
    out[i] = v;
}

// dz = g (exp(z - lse) - onehot) from the stored logits, written like the fused path's
// dlogits epilogue: token-major dz [N, ld_dz] and vocab-major dz^T [Vs, ld_dzt] in bf16,
// through a 64 x 64 LDS tile; padding columns (vocab >= Vs, token >= N) get zeros.
constexpr int kDzTile = 64;
__global__ __launch_bounds__(256) void dlogits_from_logits_kernel(
    const float *__restrict__ logits, int64_t ld, const int64_t *__restrict__ targets,
    const float *__restrict__ lse, int64_t n, int64_t start, int64_t vs, int64_t ignore_index,
    float grad_scale, uint16_t *__restrict__ dz, int64_t ld_dz, uint16_t *__restrict__ dzt,
    int64_t ld_dzt) {
    __shared__ uint16_t tile[kDzTile][kDzTile + 2];   // [token][vocab]
    const int t = threadIdx.x;
    const int64_t v0 = (int64_t)blockIdx.x * kDzTile, n0 = (int64_t)blockIdx.y * kDzTile;
    {
        const int r = t >> 2, c = (t & 3) * 16;   // token row r, vocab columns c .. c+15
        const int64_t tok = n0 + r;
        float d[16];
        if (tok < n) {
            const int64_t y = targets[tok];
            const float g = (y == ignore_index) ? 0.f : grad_scale;
            const float ll = lse[tok] * kLog2e;
            const float *row = logits + tok * ld + v0 + c;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t v = v0 + c + 4 * q;
                const f32x4 z = v < vs ? *(const f32x4 *)(row + 4 * q) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float p = fast_exp2(fmaf(z[k], kLog2e, -ll));
                    d[4 * q + k] = v + k < vs ? g * (p - (v + k == y - start ? 1.f : 0.f)) : 0.f;
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) d[k] = 0.f;
        }
        u32x4 lo, hi;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            lo[k] = (uint32_t)bf16_bits(d[2 * k]) | ((uint32_t)bf16_bits(d[2 * k + 1]) << 16);
            hi[k] = (uint32_t)bf16_bits(d[8 + 2 * k]) | ((uint32_t)bf16_bits(d[8 + 2 * k + 1]) << 16);
        }
        if (tok < n) {   // the grid covers ld_dz (a multiple of 64) exactly
            *(u32x4 *)(dz + tok * ld_dz + v0 + c) = lo;
            *(u32x4 *)(dz + tok * ld_dz + v0 + c + 8) = hi;
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) tile[r][c + k] = bf16_bits(d[k]);
    }
    __syncthreads();
    {
        const int r = t >> 2, c = (t & 3) * 16;   // vocab row r, token columns c .. c+15
        const int64_t v = v0 + r;
        if (v < vs) {   // the grid covers ld_dzt (a multiple of 64) exactly
            u32x4 lo, hi;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                lo[k] = (uint32_t)tile[c + 2 * k][r] | ((uint32_t)tile[c + 2 * k + 1][r] << 16);
                hi[k] = (uint32_t)tile[c + 8 + 2 * k][r] | ((uint32_t)tile[c + 8 + 2 * k + 1][r] << 16);
            }
            *(u32x4 *)(dzt + v * ld_dzt + n0 + c) = lo;
            *(u32x4 *)(dzt + v * ld_dzt + n0 + c + 8) = hi;
        }
    }
}

}  // namespace

hipError_t launch_lmhead_logits(const uint16_t *x, const uint16_t *w, int64_t n, int64_t h,
                                int64_t vs, float *logits, int64_t ld, hipStream_t stream) {
    // C = W_r X^T (vocab x tokens), stored transposed: logits[token, vocab]
    const GemmGrid g = gemm_grid(vs, n);
    StoreTransposedEpilogue epi{logits, ld, (int)vs, (int)n};
    hipLaunchKernelGGL(gemm_nt_kernel<StoreTransposedEpilogue>, dim3(g.blocks()), dim3(kThreads), 0,
                       stream, Operand{w, h, (int)vs}, Operand{x, h, (int)n}, (int)h, g.tiles_m,
                       g.tiles_n, epi);
    return hipGetLastError();
}

hipError_t launch_logits_stats(const float *logits, int64_t ld, const int64_t *targets, int64_t n,
                               int64_t start, int64_t vs, const float *m_ref, float *m_out,
                               float *s_out, float *zy_out, hipStream_t stream) {
    if (m_ref)
        hipLaunchKernelGGL(logits_stats_kernel<true>, dim3((unsigned)n), dim3(kStatThreads), 0, stream,
                           logits, ld, targets, start, vs, m_ref, m_out, s_out, zy_out);
    else
        hipLaunchKernelGGL(logits_stats_kernel<false>, dim3((unsigned)n), dim3(kStatThreads), 0,
                           stream, logits, ld, targets, start, vs, m_ref, m_out, s_out, zy_out);
    return hipGetLastError();
}

hipError_t launch_rows_max(const float *m, int64_t n, int T, float *out, hipStream_t stream) {
    hipLaunchKernelGGL(rows_max_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, m, n,
                       T, out);
    return hipGetLastError();
}

hipError_t launch_logits_ce_bwd(const float *logits, int64_t ld, const uint16_t *x,
                                const uint16_t *w, const int64_t *targets, const float *lse,
                                int64_t n, int64_t h, int64_t start, int64_t vs,
                                int64_t ignore_index, float grad_scale, float *dx, float *dw,
                                void *ws, hipStream_t stream) {
    if (n == 0) return launch_bwd_zero_dw(dw, vs, h, stream);
    const BwdWorkspace b = bwd_workspace(n, h, vs);
    char *base = (char *)ws;
    hipError_t e;
    if ((e = launch_bwd_transposes(x, w, n, h, vs, ws, stream)) != hipSuccess) return e;
    const dim3 grid((unsigned)(b.vs_ld / kDzTile), (unsigned)(b.n_ld / kDzTile));
    hipLaunchKernelGGL(dlogits_from_logits_kernel, grid, dim3(256), 0, stream, logits, ld, targets, lse,
                       n, start, vs, ignore_index, grad_scale, (uint16_t *)(base + b.off_dz), b.vs_ld,
                       (uint16_t *)(base + b.off_dzt), b.n_ld);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_bwd_grad_gemms(n, h, vs, dx, dw, ws, stream);
}

}  // namespace vp
