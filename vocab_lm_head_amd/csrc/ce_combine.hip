// Merge of the T shards' per-token statistics into the loss.
//
// Method: MiniMind-Tron "5 Vocab Parallelism", 5.3.1 -- the loss needs only
// the global maximum (all-reduce MAX), the global sum of exponentials
// (all-reduce SUM) and the target logit (all-reduce SUM, non-zero on the
// owner only); the interview note "Vocab parallelism" (Figure 2, key formulas)
// writes the result as loss = log S - (z_y - m).  Each shard's sum arrives
// about its own maximum, so it is rescaled by exp(m_r - m) before the sum.
// 5.3.3: ignored tokens have zero loss; the mean divides by max(1, N_valid).
//
// On one GPU this kernel replaces the three collectives; with one process per
// GPU the same kernel would run on every rank after an all-gather of the
// packed [3, n] statistics.
#include "common.hpp"
#include "launch.hpp"

namespace vp {

namespace {

// One thread per token.  The T shards' triples are read kShardBatch at a time with
// all loads of a batch in flight together; batches merge with the same
// (max, rescaled sum) rule, so any T works.
constexpr int kCombineThreads = 64;
constexpr int kShardBatch = 8;
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float *__restrict__ m, const float *__restrict__ s, const float *__restrict__ zy,
    const int64_t *__restrict__ targets, int64_t n, int T, int64_t ignore_index,
    float *__restrict__ loss, float *__restrict__ lse) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t y = targets[i];
    float M = -INFINITY, S = 0.f, Z = 0.f;
    for (int r0 = 0; r0 < T; r0 += kShardBatch) {
        float mr[kShardBatch], sr[kShardBatch], zr[kShardBatch];
#pragma unroll
        for (int u = 0; u < kShardBatch; ++u) {
            const int64_t r = r0 + u < T ? r0 + u : T - 1;
            mr[u] = m[r * n + i];
            sr[u] = s[r * n + i];
            zr[u] = zy[r * n + i];
        }
        float Mb = M;
#pragma unroll
        for (int u = 0; u < kShardBatch; ++u)
            if (r0 + u < T) Mb = fmaxf(Mb, mr[u]);
        float Sb = S != 0.f ? S * expf(M - Mb) : 0.f;
#pragma unroll
        for (int u = 0; u < kShardBatch; ++u)
            if (r0 + u < T) {
                if (sr[u] != 0.f) Sb += sr[u] * expf(mr[u] - Mb);
                Z += zr[u];
            }
        M = Mb;
        S = Sb;
    }
    const float logS = logf(S);
    lse[i] = M + logS;
    loss[i] = (y == ignore_index) ? 0.f : (logS - (Z - M));
}

// Mean over valid tokens in a fixed reduction order (one workgroup); each thread
// reads kMeanBatch tokens per round with their loads in flight together.
constexpr int kMeanThreads = 1024;
constexpr int kMeanBatch = 8;
__global__ __launch_bounds__(kMeanThreads) void mean_kernel(const float *__restrict__ loss,
                                                            const int64_t *__restrict__ targets,
                                                            int64_t n, int64_t ignore_index,
                                                            float *__restrict__ loss_mean) {
    __shared__ double ssum[kMeanThreads];
    __shared__ long long scnt[kMeanThreads];
    double acc = 0.0;
    long long cnt = 0;
    for (int64_t i0 = threadIdx.x; i0 < n; i0 += (int64_t)kMeanThreads * kMeanBatch) {
        int64_t y[kMeanBatch];
        float l[kMeanBatch];
#pragma unroll
        for (int u = 0; u < kMeanBatch; ++u) {
            const int64_t i = i0 + (int64_t)u * kMeanThreads;
            const int64_t ic = i < n ? i : n - 1;
            y[u] = targets[ic];
            l[u] = loss[ic];
        }
#pragma unroll
        for (int u = 0; u < kMeanBatch; ++u)
            if (i0 + (int64_t)u * kMeanThreads < n && y[u] != ignore_index) {
                acc += (double)l[u];
                ++cnt;
            }
    }
    ssum[threadIdx.x] = acc;
    scnt[threadIdx.x] = cnt;
    __syncthreads();
    for (int w = kMeanThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            ssum[threadIdx.x] += ssum[threadIdx.x + w];
            scnt[threadIdx.x] += scnt[threadIdx.x + w];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) loss_mean[0] = (float)(ssum[0] / (double)(scnt[0] > 0 ? scnt[0] : 1));
}

}  // namespace

hipError_t launch_ce_combine(const float *m, const float *s, const float *zy,
                             const int64_t *targets, int64_t n, int T, int64_t ignore_index,
                             float *loss, float *lse, float *loss_mean, hipStream_t stream) {
    if (n > 0)
        hipLaunchKernelGGL(combine_kernel, dim3((unsigned)ceil_div(n, kCombineThreads)),
                           dim3(kCombineThreads), 0, stream, m,
                           s, zy, targets, n, T, ignore_index, loss, lse);
    hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(kMeanThreads), 0, stream, loss, targets, n,
                       ignore_index, loss_mean);
    return hipGetLastError();
}

}  // namespace vp
