// Internal launchers behind the C ABI.  Arguments are validated by api.cpp
// before any of these is called; each returns hipGetLastError() after its
// launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vp {

// forward workspace: fp32 partial (max, sum-exp, target logit) per 128-row
// vocabulary slice and token
struct FwdWorkspace {
    int64_t slices;        // ceil(Vs / 128): per-slice partials [3][slices][n] at offset 0
    int64_t splits, chunk; // the merge's slice splits (1: a single pass) of `chunk` slices
    size_t off_split;      // per-split results [3][splits][n] when splits > 1
    size_t bytes;
};
FwdWorkspace fwd_workspace(int64_t n, int64_t vs);

// backward workspace: X^T [H, N64], W^T [H, Vs64], dz [N, Vs64], dz^T [Vs, N64] (bf16);
struct BwdWorkspace {
    int64_t n_ld, vs_ld;   // padded leading dimensions (multiples of 64)
    size_t off_xt, off_wt, off_dz, off_dzt;
    // split-K of the two gradient GEMMs (1: none) and their partials.  When both are split
    // they run as one launch (grouped) and their partials sit side by side (dX's at
    // off_split, dW's at off_split_dw); otherwise they share off_split.
    int64_t splits_dx, chunk_dx, splits_dw, chunk_dw;
    bool grouped;
    size_t off_split, off_split_dw;
    size_t bytes;
};
BwdWorkspace bwd_workspace(int64_t n, int64_t h, int64_t vs);

hipError_t launch_embed(const int64_t *ids, int64_t n, const uint16_t *w, int64_t start,
                        int64_t end, int64_t h, uint16_t *out, hipStream_t stream);

// lookup-gradient workspace: two (key, token) uint32 buffers for the radix sort's
// passes, the per-tile digit counts, and fp32 [h] partials of the rows that cross
// the segment-sum blocks (first and last row piece of each block)
struct EmbedBwdWorkspace {
    int64_t nblk;          // radix-sort tiles
    int64_t nseg;          // segment-sum blocks
    size_t off_keys[2], off_vals[2], off_hist, off_first, off_last;
    size_t bytes;
};
EmbedBwdWorkspace embed_bwd_workspace(int64_t n, int64_t h);

hipError_t launch_embed_bwd(const int64_t *ids, int64_t n, const uint16_t *dout, int64_t start,
                            int64_t vs, int64_t h, float *dw, void *ws, hipStream_t stream);

hipError_t launch_ce_fwd(const uint16_t *x, const uint16_t *w, const int64_t *targets, int64_t n,
                         int64_t h, int64_t start, int64_t vs, float *m_out, float *s_out,
                         float *zy_out, void *ws, hipStream_t stream);

// the forward with its workspace in the library's fixed per-device scratch buffer
// (caller has checked fwd_workspace(n, vs).bytes <= kNoallocScratchBytes)
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
hipError_t launch_ce_fwd_noalloc(const uint16_t *x, const uint16_t *w, const int64_t *targets,
                                 int64_t n, int64_t h, int64_t start, int64_t vs, float *m_out,
                                 float *s_out, float *zy_out, hipStream_t stream);

hipError_t launch_ce_combine(const float *m, const float *s, const float *zy,
                             const int64_t *targets, int64_t n, int T, int64_t ignore_index,
                             float *loss, float *lse, float *loss_mean, hipStream_t stream);

// pieces of the backward shared with the materialised-logits comparator: X^T and W^T into
// the workspace; the dX and dW GEMMs from the workspace's dz and dz^T; dW = 0 for n == 0
hipError_t launch_bwd_transposes(const uint16_t *x, const uint16_t *w, int64_t n, int64_t h,
                                 int64_t vs, void *ws, hipStream_t stream);
hipError_t launch_bwd_grad_gemms(int64_t n, int64_t h, int64_t vs, float *dx, float *dw, void *ws,
                                 hipStream_t stream);
hipError_t launch_bwd_zero_dw(float *dw, int64_t vs, int64_t h, hipStream_t stream);

// materialised-logits comparator
hipError_t launch_lmhead_logits(const uint16_t *x, const uint16_t *w, int64_t n, int64_t h,
                                int64_t vs, float *logits, int64_t ld, hipStream_t stream);
hipError_t launch_logits_stats(const float *logits, int64_t ld, const int64_t *targets, int64_t n,
                               int64_t start, int64_t vs, const float *m_ref, float *m_out,
                               float *s_out, float *zy_out, hipStream_t stream);
hipError_t launch_rows_max(const float *m, int64_t n, int T, float *out, hipStream_t stream);
hipError_t launch_logits_ce_bwd(const float *logits, int64_t ld, const uint16_t *x,
                                const uint16_t *w, const int64_t *targets, const float *lse,
                                int64_t n, int64_t h, int64_t start, int64_t vs,
                                int64_t ignore_index, float grad_scale, float *dx, float *dw,
                                void *ws, hipStream_t stream);

hipError_t launch_ce_bwd(const uint16_t *x, const uint16_t *w, const int64_t *targets,
                         const float *lse, int64_t n, int64_t h, int64_t start, int64_t vs,
                         int64_t ignore_index, float grad_scale, float *dx, float *dw, void *ws,
                         hipStream_t stream);

}  // namespace vp
