// One training step of the vocab-parallel LM head + cross entropy through the C ABI alone:
// device buffers from hipMalloc, a stream of its own, no torch.  For every shard t of T:
// the fused forward (vp_lmhead_ce_fwd) into row t of the [T, n] statistics; then the merge
// (vp_ce_combine); then every shard's backward (vp_lmhead_ce_bwd) with the mean loss's
// upstream gradient 1 / max(1, N_valid).
//
//   vp_step <in.bin> <out.bin>
//   in.bin : int64 n, h, V, T, ignore_index; bf16 x [n, h]; bf16 w [V, h]; int64 targets [n]
//   out.bin: fp32 loss [n], lse [n], mean [1], dx [T][n, h] (each shard's partial),
//            dw [V, h] (the shards' gradients, stacked)
// Exit status 0 on success; otherwise the failing call and its status string are printed.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

#include "vp_lmhead.h"

#define HIP_OK(x)                                                                       \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
            std::exit(2);                                                               \
        }                                                                               \
    } while (0)
#define VP_OK_(x)                                                                       \
    do {                                                                                \
        int s_ = (x);                                                                   \
        if (s_ != VP_OK) {                                                              \
            std::fprintf(stderr, "%s: %s\n", #x, vp_status_string(s_));                \
            std::exit(3);                                                               \
        }                                                                               \
    } while (0)

template <class T>
static void read_n(std::FILE *f, T *p, size_t n) {
    if (std::fread(p, sizeof(T), n, f) != n) {
        std::fprintf(stderr, "short input file\n");
        std::exit(4);
    }
}

template <class T>
static T *to_device(const std::vector<T> &v) {
    T *d = nullptr;
    HIP_OK(hipMalloc(&d, v.size() * sizeof(T) + 16));
    HIP_OK(hipMemcpy(d, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice));
    return d;
}

int main(int argc, char **argv) {
    if (argc != 3) {
        std::fprintf(stderr, "usage: %s <in.bin> <out.bin>\n", argv[0]);
        return 1;
    }
    std::FILE *fi = std::fopen(argv[1], "rb");
    if (!fi) {
        std::perror(argv[1]);
        return 1;
    }
    int64_t hdr[5];
    read_n(fi, hdr, 5);
    const int64_t n = hdr[0], h = hdr[1], V = hdr[2], ignore = hdr[4];
    const int32_t T = (int32_t)hdr[3];
    std::vector<uint16_t> x((size_t)(n * h)), w((size_t)(V * h));
    std::vector<int64_t> y((size_t)n);
    read_n(fi, x.data(), x.size());
    read_n(fi, w.data(), w.size());
    read_n(fi, y.data(), y.size());
    std::fclose(fi);
    int64_t valid = 0;
    for (int64_t t : y) valid += t != ignore;
    const float grad_scale = 1.0f / (float)(valid > 1 ? valid : 1);

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));   // default priority
    uint16_t *dx_in = to_device(x), *dw_in = to_device(w);
    int64_t *dy = to_device(y);
    float *m, *s, *zy, *loss, *lse, *mean, *dx, *dw;
    HIP_OK(hipMalloc(&m, (size_t)T * n * 4));
    HIP_OK(hipMalloc(&s, (size_t)T * n * 4));
    HIP_OK(hipMalloc(&zy, (size_t)T * n * 4));
    HIP_OK(hipMalloc(&loss, (size_t)n * 4));
    HIP_OK(hipMalloc(&lse, (size_t)n * 4));
    HIP_OK(hipMalloc(&mean, 4));
    HIP_OK(hipMalloc(&dx, (size_t)T * n * h * 4));
    HIP_OK(hipMalloc(&dw, (size_t)V * h * 4));

    std::vector<void *> workspaces;
    auto workspace = [&](size_t bytes) {
        void *p = nullptr;
        HIP_OK(hipMalloc(&p, bytes > 0 ? bytes : 1));   // hipMalloc memory is 256-byte aligned
        workspaces.push_back(p);
        return p;
    };
    for (int32_t t = 0; t < T; ++t) {
        int64_t lo, hi;
        VP_OK_(vp_shard_range(V, T, t, &lo, &hi));
        const size_t wb = vp_lmhead_ce_fwd_workspace(n, h, lo, hi);
        VP_OK_(vp_lmhead_ce_fwd(dx_in, dw_in + lo * h, dy, n, h, lo, hi, m + (size_t)t * n,
                                s + (size_t)t * n, zy + (size_t)t * n, workspace(wb), wb, stream));
    }
    VP_OK_(vp_ce_combine(m, s, zy, dy, n, T, ignore, loss, lse, mean, stream));
    for (int32_t t = 0; t < T; ++t) {
        int64_t lo, hi;
        VP_OK_(vp_shard_range(V, T, t, &lo, &hi));
        const size_t wb = vp_lmhead_ce_bwd_workspace(n, h, lo, hi);
        VP_OK_(vp_lmhead_ce_bwd(dx_in, dw_in + lo * h, dy, lse, n, h, lo, hi, ignore, grad_scale,
                                dx + (size_t)t * n * h, dw + lo * h, workspace(wb), wb, stream));
    }
    HIP_OK(hipStreamSynchronize(stream));

    std::vector<float> out((size_t)(2 * n + 1 + T * n * h + V * h));
    float *o = out.data();
    HIP_OK(hipMemcpy(o, loss, (size_t)n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(o + n, lse, (size_t)n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(o + 2 * n, mean, 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(o + 2 * n + 1, dx, (size_t)T * n * h * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(o + 2 * n + 1 + T * n * h, dw, (size_t)V * h * 4, hipMemcpyDeviceToHost));
    std::FILE *fo = std::fopen(argv[2], "wb");
    if (!fo || std::fwrite(out.data(), 4, out.size(), fo) != out.size()) {
        std::perror(argv[2]);
        return 1;
    }
    std::fclose(fo);
    for (void *p : workspaces) HIP_OK(hipFree(p));
    for (void *p : {(void *)dx_in, (void *)dw_in, (void *)dy, (void *)m, (void *)s, (void *)zy,
                    (void *)loss, (void *)lse, (void *)mean, (void *)dx, (void *)dw})
        HIP_OK(hipFree(p));
    HIP_OK(hipStreamDestroy(stream));
    std::printf("vp_step: n=%lld h=%lld V=%lld T=%d ok\n", (long long)n, (long long)h, (long long)V, T);
    return 0;
}
