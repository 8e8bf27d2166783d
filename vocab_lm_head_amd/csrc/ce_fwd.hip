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
#include <algorithm>
#include <mutex>

#include "gemm.hpp"
#include "launch.hpp"

// Fixed scratch of the allocation-free forward (vp_lmhead_ce_fwd_noalloc): each GPU the
// library runs on holds one copy, at an address of its own, until the process ends.  In
// host code this name is not a device address; the address of each GPU's copy comes from
// hipGetSymbolAddress with that GPU current (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[vp::kNoallocScratchBytes];

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
            // The target's row relative to this lane's first row is 16 it + rt, with rt < 4,
            // for at most one lane of the column, and never when the target lies outside the
            // shard: pick MFMA tile it, then its component rt.  (The asm keeps the compiler
            // from splitting the range test into every comparison.)
            const int64_t local = tg[j] - start;
            int tr = (local >= 0 && local < M) ? (int)(local - mbase) - rsub : -1;
            asm volatile("" : "+v"(tr));
            const int it = tr >> 4, rt = tr & 15;
            f32x4 t4 = acc[0][j];
#pragma unroll
            for (int i = 1; i < kTM; ++i) t4 = (it == i) ? acc[i][j] : t4;
            const float z = rt == 0 ? t4[0] : rt == 1 ? t4[1] : rt == 2 ? t4[2] : t4[3];
            zy[j] = (tr >= 0 && tr < kWM && rt < 4) ? z : 0.f;
            // the sum of exponentials about the column maximum, in two interleaved partial
            // sums (two independent dependency chains)
            const float mxl = mx[j] * kLog2e;
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int i = 0; i < kTM; ++i) {
                s0 += fast_exp2(fmaf(acc[i][j][0], kLog2e, -mxl));
                s1 += fast_exp2(fmaf(acc[i][j][1], kLog2e, -mxl));
                s0 += fast_exp2(fmaf(acc[i][j][2], kLog2e, -mxl));
                s1 += fast_exp2(fmaf(acc[i][j][3], kLog2e, -mxl));
            }
            sum[j] = s0 + s1;
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

// Merge the shard's per-slice partials of each token.  A workgroup takes 32 tokens
// and the slices [blockIdx.y chunk, (blockIdx.y + 1) chunk); its 8 thread groups each
// merge every 8th of them, kMergeBatch slices at a time with all of their loads issued
// before the first is used, then the 8 partial results are merged through LDS and
// written at row blockIdx.y of the outputs (rows out_stride apart).  The input and the
// output rows share one layout, [3][rows][n] (max, sum-exp, target logit), so the
// same kernel merges the per-split results of a first pass.
constexpr int kMergeTok = 32, kMergeGrp = 8, kMergeBatch = 16;
__global__ __launch_bounds__(kMergeTok * kMergeGrp) void merge_slices_kernel(
    const float *__restrict__ part, int64_t slices, int64_t n, int64_t chunk,
    float *__restrict__ m_out, float *__restrict__ s_out, float *__restrict__ zy_out,
    int64_t out_stride) {
    __shared__ float sm[kMergeGrp][kMergeTok], ss[kMergeGrp][kMergeTok], sz[kMergeGrp][kMergeTok];
    const int t = threadIdx.x % kMergeTok, g = threadIdx.x / kMergeTok;
    const int64_t i = (int64_t)blockIdx.x * kMergeTok + t;
    const int64_t ic = i < n ? i : n - 1;   // past n: a valid address, result unused
    const int64_t p_lo = (int64_t)blockIdx.y * chunk, p_hi = min(p_lo + chunk, slices);
    float m = -INFINITY, s = 0.f, zy = 0.f;
    for (int64_t p0 = p_lo + g; p0 < p_hi; p0 += kMergeGrp * kMergeBatch) {
        float mp[kMergeBatch], sp[kMergeBatch], zp[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            const int64_t p = p0 + u * kMergeGrp;
            const int64_t pc = p < p_hi ? p : p_hi - 1;
            mp[u] = part[pc * n + ic];
            sp[u] = part[(slices + pc) * n + ic];
            zp[u] = part[(2 * slices + pc) * n + ic];
        }
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            if (p0 + u * kMergeGrp >= p_hi) break;
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
        const int64_t o = (int64_t)blockIdx.y * out_stride + i;
        m_out[o] = M;
        s_out[o] = S;
        zy_out[o] = Z;
    }
}

// The slices are split over more workgroups (a first pass whose per-split results a
// second pass merges) when one workgroup per 32 tokens would leave most of the chip idle
// (fewer than kMergeMinBlocks of them: aim for kMergeTargetBlocks) or would walk more
// than kMergeMaxSlices slices each.
constexpr int64_t kMergeMinBlocks = 256;
constexpr int64_t kMergeTargetBlocks = 1024;
constexpr int64_t kMergeMaxSlices = 256;

}  // namespace

FwdWorkspace fwd_workspace(int64_t n, int64_t vs) {
    FwdWorkspace w;
    w.slices = ceil_div(vs, kSlice);
    const int64_t tb = ceil_div(n, kMergeTok);
    w.splits = ceil_div(w.slices, kMergeMaxSlices);
    if (tb > 0 && tb < kMergeMinBlocks) {
        const int64_t most = std::max<int64_t>(1, w.slices / (kMergeGrp * kMergeBatch));
        w.splits = std::max(w.splits, std::min(ceil_div(kMergeTargetBlocks, tb), most));
    }
    w.chunk = ceil_div(w.slices, w.splits);
    w.splits = ceil_div(w.slices, w.chunk);   // no empty split
    w.off_split = (size_t)round_up(3 * w.slices * n * (int64_t)sizeof(float), 256);
    w.bytes = w.off_split +
              (w.splits > 1 ? (size_t)round_up(3 * w.splits * n * (int64_t)sizeof(float), 256) : 0);
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
    const unsigned tb = (unsigned)ceil_div(n, kMergeTok);
    if (fw.splits == 1) {
        hipLaunchKernelGGL(merge_slices_kernel, dim3(tb), dim3(kMergeTok * kMergeGrp), 0, stream, part,
                           fw.slices, n, fw.slices, m_out, s_out, zy_out, (int64_t)0);
    } else {
        float *p2 = (float *)((char *)ws + fw.off_split);   // [3][splits][n]
        hipLaunchKernelGGL(merge_slices_kernel, dim3(tb, (unsigned)fw.splits),
                           dim3(kMergeTok * kMergeGrp), 0, stream, part, fw.slices, n, fw.chunk, p2,
                           p2 + fw.splits * n, p2 + 2 * fw.splits * n, n);
        hipLaunchKernelGGL(merge_slices_kernel, dim3(tb), dim3(kMergeTok * kMergeGrp), 0, stream, p2,
                           fw.splits, n, fw.splits, m_out, s_out, zy_out, (int64_t)0);
    }
    return hipGetLastError();
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];   // per device: its copy of `scratch`, once looked up

// Device address of the scratch copy on the GPU that `stream` runs on; looked up once per
// GPU, with that GPU current (the caller's current device is restored).
hipError_t noalloc_scratch(hipStream_t stream, void **out) {
    hipDevice_t dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess) return e;
        if (back != hipSuccess) return back;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

hipError_t launch_ce_fwd_noalloc(const uint16_t *x, const uint16_t *w, const int64_t *targets,
                                 int64_t n, int64_t h, int64_t start, int64_t vs, float *m_out,
                                 float *s_out, float *zy_out, hipStream_t stream) {
    void *ws = nullptr;
    const hipError_t e = noalloc_scratch(stream, &ws);
    if (e != hipSuccess) return e;
    return launch_ce_fwd(x, w, targets, n, h, start, vs, m_out, s_out, zy_out, ws, stream);
}

}  // namespace vp
