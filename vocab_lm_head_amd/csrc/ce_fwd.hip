// Fused LM-head forward of one vocabulary shard: z = W_r X^T on MFMA, with the
// cross-entropy statistics taken from the accumulators in registers.
//
// Method: MiniMind-Tron "5 Vocab Parallelism", 5.3.1 -- per token, each shard
// needs only its local maximum, its sum of exponentials and the target logit
// if it owns the target (interview note "Vocab parallelism", Figure 2).  Here
// the sum is taken about the shard's own maximum in a single pass, and the
// shard's 128-row vocabulary slices are merged with
//   (m, s) <- (max(m, m'), s e^(m - max) + s' e^(m' - max)),
// which is exact in real arithmetic; the [N, Vs] logits never leave registers.
#include "gemm.hpp"
#include "launch.hpp"

namespace vp {

namespace {

constexpr int kSlice = kWM;   // vocabulary rows per partial = one wave tile

struct CeStatsEpilogue {
    const int64_t *targets;
    int64_t start;        // vocab_start
    int M;                // Vs
    int N;                // tokens
    float *part;          // [3][slices][N]: max, sum-exp, target logit
    int64_t slices;

    __device__ __forceinline__ void operator()(Acc &acc, int mbase, int nbase, int lane, int, int,
                                               uint16_t *) const {
        if (mbase >= M) return;                   // wave tile entirely past the shard
        const bool full = mbase + kWM <= M;
        const int rsub = 4 * (lane >> 4);
        const int64_t p = mbase / kSlice;
        float *pm = part + p * N;
        float *ps = part + (slices + p) * N;
        float *pz = part + (2 * slices + p) * N;
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            const int n = nbase + 16 * j + (lane & 15);
            // target row relative to this wave tile; -1 unless the target lies in the shard
            // (rows past the shard's end exist in the last tile but hold no shard data)
            int64_t trow = -1;
            if (n < N) {
                const int64_t local = targets[n] - start;
                if (local >= 0 && local < M) trow = local - mbase;
            }
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * i + rsub + r;
                    if (full || mbase + row < M) mx = fmaxf(mx, acc[i][j][r]);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mxl = mx * kLog2e;
            float s = 0.f, zy = 0.f;
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * i + rsub + r;
                    const float v = acc[i][j][r];
                    if (full || mbase + row < M) s += fast_exp2(fmaf(v, kLog2e, -mxl));
                    if (row == trow) zy = v;
                }
            s += __shfl_xor(s, 16);
            s += __shfl_xor(s, 32);
            zy += __shfl_xor(zy, 16);
            zy += __shfl_xor(zy, 32);
            if (lane < 16 && n < N) {
                pm[n] = mx;
                ps[n] = s;
                pz[n] = zy;
            }
        }
    }
};

// Merge the shard's per-slice partials of each token.  A workgroup takes 32
// tokens; its 8 thread groups each merge every 8th slice (independent loads
// in flight), then the 8 partial results are merged through LDS.
constexpr int kMergeTok = 32, kMergeGrp = 8;
__global__ __launch_bounds__(kMergeTok * kMergeGrp) void merge_slices_kernel(
    const float *__restrict__ part, int64_t slices, int64_t n, float *__restrict__ m_out,
    float *__restrict__ s_out, float *__restrict__ zy_out) {
    __shared__ float sm[kMergeGrp][kMergeTok], ss[kMergeGrp][kMergeTok], sz[kMergeGrp][kMergeTok];
    const int t = threadIdx.x % kMergeTok, g = threadIdx.x / kMergeTok;
    const int64_t i = (int64_t)blockIdx.x * kMergeTok + t;
    float m = -INFINITY, s = 0.f, zy = 0.f;
    if (i < n) {
        for (int64_t p = g; p < slices; p += kMergeGrp) {
            const float mp = part[p * n + i];
            const float sp = part[(slices + p) * n + i];
            zy += part[(2 * slices + p) * n + i];
            const float mx = fmaxf(m, mp);
            s = s * fast_exp2((m - mx) * kLog2e) + sp * fast_exp2((mp - mx) * kLog2e);
            m = mx;
        }
    }
    sm[g][t] = m;
    ss[g][t] = s;
    sz[g][t] = zy;
    __syncthreads();
    if (g == 0 && i < n) {
        float M = -INFINITY;
        for (int q = 0; q < kMergeGrp; ++q) M = fmaxf(M, sm[q][t]);
        float S = 0.f, Z = 0.f;
        for (int q = 0; q < kMergeGrp; ++q) {
            if (ss[q][t] != 0.f) S += ss[q][t] * fast_exp2((sm[q][t] - M) * kLog2e);
            Z += sz[q][t];
        }
        m_out[i] = M;
        s_out[i] = S;
        zy_out[i] = Z;
    }
}

}  // namespace

FwdWorkspace fwd_workspace(int64_t n, int64_t vs) {
    FwdWorkspace w;
    w.slices = ceil_div(vs, kSlice);
    w.bytes = (size_t)round_up(3 * w.slices * n * (int64_t)sizeof(float), 256);
    return w;
}

hipError_t launch_ce_fwd(const uint16_t *x, const uint16_t *w, const int64_t *targets, int64_t n,
                         int64_t h, int64_t start, int64_t vs, float *m_out, float *s_out,
                         float *zy_out, void *ws, hipStream_t stream) {
    const FwdWorkspace fw = fwd_workspace(n, vs);
    float *part = (float *)ws;
    const GemmGrid g = gemm_grid(vs, n);
    CeStatsEpilogue epi{targets, start, (int)vs, (int)n, part, fw.slices};
    Operand A{w, h, (int)vs};
    Operand B{x, h, (int)n};
    hipLaunchKernelGGL(gemm_nt_kernel<CeStatsEpilogue>, dim3(g.blocks()), dim3(kThreads), 0, stream,
                       A, B, (int)h, g.tiles_m, g.tiles_n, epi);
    hipLaunchKernelGGL(merge_slices_kernel, dim3((unsigned)ceil_div(n, kMergeTok)),
                       dim3(kMergeTok * kMergeGrp), 0, stream, part, fw.slices, n, m_out, s_out, zy_out);
    return hipGetLastError();
}

}  // namespace vp
