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
        const int rsub = 4 * (lane >> 4);
        const int64_t p = mbase / kSlice;
        float *pm = part + p * N;
        float *ps = part + (slices + p) * N;
        float *pz = part + (2 * slices + p) * N;
        // all of this lane's targets are loaded before any is used: one memory latency
        // per tile; columns past N read token N-1 and are not stored
        int64_t tg[kTN];
#pragma unroll
        for (int j = 0; j < kTN; ++j) tg[j] = targets[min(nbase + 16 * j + (lane & 15), N - 1)];
        __builtin_amdgcn_sched_barrier(0);
        // rows past the shard's end (only in its last tile; a wave-uniform branch)
        // hold no shard data: -inf drops them from the max and the sum
        if (mbase + kWM > M) {
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (mbase + 16 * i + rsub + r >= M)
#pragma unroll
                        for (int j = 0; j < kTN; ++j) acc[i][j][r] = -INFINITY;
        }
        // per column: the lane's 32 rows, then the 4 lanes sharing the column
        float mx[kTN];
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            float a = acc[0][j][0];
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) a = fmaxf(a, acc[i][j][r]);
            mx[j] = a;
        }
#pragma unroll
        for (int j = 0; j < kTN; ++j) mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], 16));
#pragma unroll
        for (int j = 0; j < kTN; ++j) mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], 32));
        float sum[kTN], zy[kTN];
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            // target row relative to this lane's first row; matches 16 i + r for at most
            // one (i, r), and never when the target lies outside the shard
            const int64_t local = tg[j] - start;
            const int tr = (local >= 0 && local < M) ? (int)(local - mbase) - rsub : -1;
            const float mxl = mx[j] * kLog2e;
            float sj = 0.f, zj = 0.f;
#pragma unroll
            for (int i = 0; i < kTM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v = acc[i][j][r];
                    sj += fast_exp2(fmaf(v, kLog2e, -mxl));
                    zj = (tr == 16 * i + r) ? v : zj;
                }
            sum[j] = sj;
            zy[j] = zj;
        }
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            sum[j] += __shfl_xor(sum[j], 16);
            zy[j] += __shfl_xor(zy[j], 16);
        }
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            sum[j] += __shfl_xor(sum[j], 32);
            zy[j] += __shfl_xor(zy[j], 32);
        }
        if (lane < 16) {
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const int n = nbase + 16 * j + lane;
                if (n < N) {
                    pm[n] = mx[j];
                    ps[n] = sum[j];
                    pz[n] = zy[j];
                }
            }
        }
    }
};

// Merge the shard's per-slice partials of each token.  A workgroup takes 32
// tokens; its 8 thread groups each merge every 8th slice, kMergeBatch slices at a
// time with all of their loads issued before the first is used, then the 8
// partial results are merged through LDS.
constexpr int kMergeTok = 32, kMergeGrp = 8, kMergeBatch = 4;
__global__ __launch_bounds__(kMergeTok * kMergeGrp) void merge_slices_kernel(
    const float *__restrict__ part, int64_t slices, int64_t n, float *__restrict__ m_out,
    float *__restrict__ s_out, float *__restrict__ zy_out) {
    __shared__ float sm[kMergeGrp][kMergeTok], ss[kMergeGrp][kMergeTok], sz[kMergeGrp][kMergeTok];
    const int t = threadIdx.x % kMergeTok, g = threadIdx.x / kMergeTok;
    const int64_t i = (int64_t)blockIdx.x * kMergeTok + t;
    const int64_t ic = i < n ? i : n - 1;   // past n: a valid address, result unused
    float m = -INFINITY, s = 0.f, zy = 0.f;
    for (int64_t p0 = g; p0 < slices; p0 += kMergeGrp * kMergeBatch) {
        float mp[kMergeBatch], sp[kMergeBatch], zp[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            const int64_t p = p0 + u * kMergeGrp;
            const int64_t pc = p < slices ? p : slices - 1;
            mp[u] = part[pc * n + ic];
            sp[u] = part[(slices + pc) * n + ic];
            zp[u] = part[(2 * slices + pc) * n + ic];
        }
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            if (p0 + u * kMergeGrp >= slices) break;
            const float mx = fmaxf(m, mp[u]);
            s = s * fast_exp2((m - mx) * kLog2e) + sp[u] * fast_exp2((mp[u] - mx) * kLog2e);
            m = mx;
            zy += zp[u];
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
