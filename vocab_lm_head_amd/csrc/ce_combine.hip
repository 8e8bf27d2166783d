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

__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ m,
                                                      const float *__restrict__ s,
                                                      const float *__restrict__ zy,
                                                      const int64_t *__restrict__ targets,
                                                      int64_t n, int T, int64_t ignore_index,
                                                      float *__restrict__ loss,
                                                      float *__restrict__ lse) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float M = -INFINITY;
    for (int r = 0; r < T; ++r) M = fmaxf(M, m[(int64_t)r * n + i]);
    float S = 0.f, Z = 0.f;
    for (int r = 0; r < T; ++r) {
        const float mr = m[(int64_t)r * n + i];
        const float sr = s[(int64_t)r * n + i];
        if (sr != 0.f) S += sr * expf(mr - M);
        Z += zy[(int64_t)r * n + i];
    }
    const float logS = logf(S);
    lse[i] = M + logS;
    loss[i] = (targets[i] == ignore_index) ? 0.f : (logS - (Z - M));
}

// Mean over valid tokens in a fixed reduction order (one workgroup).
constexpr int kMeanThreads = 1024;
__global__ __launch_bounds__(kMeanThreads) void mean_kernel(const float *__restrict__ loss,
                                                            const int64_t *__restrict__ targets,
                                                            int64_t n, int64_t ignore_index,
                                                            float *__restrict__ loss_mean) {
    __shared__ double ssum[kMeanThreads];
    __shared__ long long scnt[kMeanThreads];
    double acc = 0.0;
    long long cnt = 0;
    for (int64_t i = threadIdx.x; i < n; i += kMeanThreads) {
        if (targets[i] != ignore_index) {
            acc += (double)loss[i];
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
        hipLaunchKernelGGL(combine_kernel, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, stream, m,
                           s, zy, targets, n, T, ignore_index, loss, lse);
    hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(kMeanThreads), 0, stream, loss, targets, n,
                       ignore_index, loss_mean);
    return hipGetLastError();
}

}  // namespace vp
