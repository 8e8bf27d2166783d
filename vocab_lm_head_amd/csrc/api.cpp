// C ABI of the vocab-parallel LM head + cross entropy (declared in include/vp_lmhead.h).
//
// Every entry point validates its arguments on the host, before anything is
// launched, then enqueues its kernels on the caller's stream and returns
// without synchronising.  No exception crosses this boundary.
#include "vp_lmhead.h"

#include <stdint.h>

#include "launch.hpp"

namespace {

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Shared checks of a (hidden, weight shard) pair.
int check_shard(int64_t n, int64_t h, int64_t vocab_start, int64_t vocab_end) {
    if (n < 0 || h <= 0) return VP_ERR_SHAPE;
    if (vocab_start < 0 || vocab_end <= vocab_start) return VP_ERR_RANGE;
    // the GEMMs address 256-row operand panels through 1 GiB buffer resources, and
    // every operand row (H, N or Vs elements, padded) must stay below 2M elements
    if (n > (1 << 20) || h > (1 << 20) || vocab_end - vocab_start > (1 << 20))
        return VP_ERR_SHAPE;
    if (h % 8 != 0) return VP_ERR_ALIGN;
    return VP_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? VP_OK : VP_ERR_HIP; }

// stored logits: the fp32 store epilogue addresses 256 token rows of ld elements through
// one 1 GiB buffer resource
constexpr int64_t kMaxLogitsLd = ((int64_t)1 << 20) + 1024;

// lookup gradient: token indices and sorted positions are 32-bit, and a shard's
// row keys (plus the off-shard key) must fit 31 bits
constexpr int64_t kEmbedBwdMaxN = (int64_t)1 << 24;
constexpr int64_t kEmbedBwdMaxRows = ((int64_t)1 << 31) - 1;

}  // namespace

extern "C" {

const char *vp_status_string(int status) {
    switch (status) {
        case VP_OK: return "VP_OK";
        case VP_ERR_NULL: return "VP_ERR_NULL: a required pointer is null";
        case VP_ERR_SHAPE: return "VP_ERR_SHAPE: invalid size (negative, zero, too large, or V % T != 0)";
        case VP_ERR_RANGE: return "VP_ERR_RANGE: invalid vocabulary interval or shard index";
        case VP_ERR_ALIGN: return "VP_ERR_ALIGN: h must be a multiple of 8 and tensors 16-byte aligned";
        case VP_ERR_WORKSPACE: return "VP_ERR_WORKSPACE: workspace missing or too small";
        case VP_ERR_HIP: return "VP_ERR_HIP: the HIP runtime reported a launch error";
        case VP_ERR_SCRATCH:
            return "VP_ERR_SCRATCH: the call needs more than the allocation-free entry point's "
                   "fixed scratch buffer (VP_NOALLOC_SCRATCH_BYTES); use the workspace form";
        default: return "unknown vp_status";
    }
}

int vp_shard_range(int64_t V, int32_t T, int32_t t, int64_t *start, int64_t *end) {
    if (!start || !end) return VP_ERR_NULL;
    if (V <= 0 || T < 1 || V % T != 0) return VP_ERR_SHAPE;
    if (t < 0 || t >= T) return VP_ERR_RANGE;
    const int64_t vs = V / T;
    *start = (int64_t)t * vs;
    *end = *start + vs;
    return VP_OK;
}

int vp_padded_vocab(int64_t V, int32_t T, int64_t multiple, int64_t *V_pad) {
    if (!V_pad) return VP_ERR_NULL;
    if (V <= 0 || T < 1 || multiple < 1 || multiple > INT64_MAX / T) return VP_ERR_SHAPE;
    const int64_t q = multiple * T;
    if (V > INT64_MAX - (q - 1)) return VP_ERR_SHAPE;
    *V_pad = (V + q - 1) / q * q;
    return VP_OK;
}

int vp_embed_fwd(const int64_t *ids, int64_t n, const uint16_t *w_shard, int64_t vocab_start,
                 int64_t vocab_end, int64_t h, uint16_t *out, hipStream_t stream) {
    if (n < 0 || h <= 0) return VP_ERR_SHAPE;
    if (vocab_start < 0 || vocab_end <= vocab_start) return VP_ERR_RANGE;
    if (h % 8 != 0) return VP_ERR_ALIGN;
    if (n == 0) return VP_OK;
    if (!ids || !w_shard || !out) return VP_ERR_NULL;
    if (!aligned(ids, 8) || !aligned(w_shard, 16) || !aligned(out, 16)) return VP_ERR_ALIGN;
    return hip_status(vp::launch_embed(ids, n, w_shard, vocab_start, vocab_end, h, out, stream));
}

size_t vp_embed_bwd_workspace(int64_t n, int64_t h, int64_t vocab_start, int64_t vocab_end) {
    if (n <= 0 || n > kEmbedBwdMaxN || h <= 0 || h % 8 != 0 || vocab_start < 0 ||
        vocab_end <= vocab_start || vocab_end - vocab_start > kEmbedBwdMaxRows)
        return 0;
    return vp::embed_bwd_workspace(n, h).bytes;
}

int vp_embed_bwd(const int64_t *ids, int64_t n, const uint16_t *dout, int64_t vocab_start,
                 int64_t vocab_end, int64_t h, float *dw, void *workspace, size_t workspace_bytes,
                 hipStream_t stream) {
    if (n < 0 || h <= 0 || n > kEmbedBwdMaxN) return VP_ERR_SHAPE;
    if (vocab_start < 0 || vocab_end <= vocab_start) return VP_ERR_RANGE;
    if (vocab_end - vocab_start > kEmbedBwdMaxRows) return VP_ERR_SHAPE;
    if (h % 8 != 0) return VP_ERR_ALIGN;
    if (n == 0) return VP_OK;
    if (!ids || !dout || !dw) return VP_ERR_NULL;
    if (!aligned(ids, 8) || !aligned(dout, 16) || !aligned(dw, 16)) return VP_ERR_ALIGN;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < vp::embed_bwd_workspace(n, h).bytes)
        return VP_ERR_WORKSPACE;
    return hip_status(vp::launch_embed_bwd(ids, n, dout, vocab_start, vocab_end - vocab_start, h, dw,
                                           workspace, stream));
}

size_t vp_lmhead_ce_fwd_workspace(int64_t n, int64_t h, int64_t vocab_start, int64_t vocab_end) {
    if (check_shard(n, h, vocab_start, vocab_end) != VP_OK || n == 0) return 0;
    return vp::fwd_workspace(n, vocab_end - vocab_start).bytes;
}

int vp_lmhead_ce_fwd(const uint16_t *hidden, const uint16_t *w_shard, const int64_t *targets,
                     int64_t n, int64_t h, int64_t vocab_start, int64_t vocab_end, float *m_local,
                     float *s_local, float *zy_local, void *workspace, size_t workspace_bytes,
                     hipStream_t stream) {
    int st = check_shard(n, h, vocab_start, vocab_end);
    if (st != VP_OK) return st;
    if (n == 0) return VP_OK;
    if (!hidden || !w_shard || !targets || !m_local || !s_local || !zy_local) return VP_ERR_NULL;
    if (!aligned(hidden, 16) || !aligned(w_shard, 16) || !aligned(targets, 8) ||
        !aligned(m_local, 4) || !aligned(s_local, 4) || !aligned(zy_local, 4))
        return VP_ERR_ALIGN;
    const int64_t vs = vocab_end - vocab_start;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < vp::fwd_workspace(n, vs).bytes)
        return VP_ERR_WORKSPACE;
    return hip_status(vp::launch_ce_fwd(hidden, w_shard, targets, n, h, vocab_start, vs, m_local,
                                        s_local, zy_local, workspace, stream));
}

int vp_lmhead_ce_fwd_noalloc(const uint16_t *hidden, const uint16_t *w_shard,
                             const int64_t *targets, int64_t n, int64_t h, int64_t vocab_start,
                             int64_t vocab_end, float *m_local, float *s_local, float *zy_local,
                             hipStream_t stream) {
    static_assert(VP_NOALLOC_SCRATCH_BYTES == vp::kNoallocScratchBytes, "one scratch size");
    int st = check_shard(n, h, vocab_start, vocab_end);
    if (st != VP_OK) return st;
    if (n == 0) return VP_OK;
    if (!hidden || !w_shard || !targets || !m_local || !s_local || !zy_local) return VP_ERR_NULL;
    if (!aligned(hidden, 16) || !aligned(w_shard, 16) || !aligned(targets, 8) ||
        !aligned(m_local, 4) || !aligned(s_local, 4) || !aligned(zy_local, 4))
        return VP_ERR_ALIGN;
    const int64_t vs = vocab_end - vocab_start;
    if (vp::fwd_workspace(n, vs).bytes > vp::kNoallocScratchBytes) return VP_ERR_SCRATCH;
    return hip_status(vp::launch_ce_fwd_noalloc(hidden, w_shard, targets, n, h, vocab_start, vs,
                                                m_local, s_local, zy_local, stream));
}

int vp_ce_combine(const float *m, const float *s, const float *zy, const int64_t *targets,
                  int64_t n, int32_t T, int64_t ignore_index, float *loss, float *lse,
                  float *loss_mean, hipStream_t stream) {
    // one thread per token: n is capped so that the grid stays far inside its limits
    if (n < 0 || T < 1 || n > ((int64_t)1 << 31) || n > INT64_MAX / T) return VP_ERR_SHAPE;
    if (!loss_mean) return VP_ERR_NULL;
    if (n > 0) {
        if (!m || !s || !zy || !targets || !loss || !lse) return VP_ERR_NULL;
        if (!aligned(m, 4) || !aligned(s, 4) || !aligned(zy, 4) || !aligned(targets, 8) ||
            !aligned(loss, 4) || !aligned(lse, 4))
            return VP_ERR_ALIGN;
    }
    if (!aligned(loss_mean, 4)) return VP_ERR_ALIGN;
    return hip_status(
        vp::launch_ce_combine(m, s, zy, targets, n, T, ignore_index, loss, lse, loss_mean, stream));
}

size_t vp_lmhead_ce_bwd_workspace(int64_t n, int64_t h, int64_t vocab_start, int64_t vocab_end) {
    if (check_shard(n, h, vocab_start, vocab_end) != VP_OK || n == 0) return 0;
    return vp::bwd_workspace(n, h, vocab_end - vocab_start).bytes;
}

int vp_lmhead_ce_bwd(const uint16_t *hidden, const uint16_t *w_shard, const int64_t *targets,
                     const float *lse, int64_t n, int64_t h, int64_t vocab_start,
                     int64_t vocab_end, int64_t ignore_index, float grad_scale, float *dx,
                     float *dw, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    int st = check_shard(n, h, vocab_start, vocab_end);
    if (st != VP_OK) return st;
    const int64_t vs = vocab_end - vocab_start;
    if (!dw) return VP_ERR_NULL;
    if (!aligned(dw, 16)) return VP_ERR_ALIGN;
    if (n > 0) {
        if (!hidden || !w_shard || !targets || !lse || !dx) return VP_ERR_NULL;
        if (!aligned(hidden, 16) || !aligned(w_shard, 16) || !aligned(targets, 8) ||
            !aligned(lse, 4) || !aligned(dx, 16))
            return VP_ERR_ALIGN;
        if (!workspace || !aligned(workspace, 256) ||
            workspace_bytes < vp::bwd_workspace(n, h, vs).bytes)
            return VP_ERR_WORKSPACE;
    }
    return hip_status(vp::launch_ce_bwd(hidden, w_shard, targets, lse, n, h, vocab_start, vs,
                                        ignore_index, grad_scale, dx, dw, workspace, stream));
}

// ---- materialised-logits comparator ----------------------------------------------------

int vp_lmhead_logits(const uint16_t *hidden, const uint16_t *w_shard, int64_t n, int64_t h,
                     int64_t vocab_start, int64_t vocab_end, float *logits, int64_t ld_logits,
                     hipStream_t stream) {
    int st = check_shard(n, h, vocab_start, vocab_end);
    if (st != VP_OK) return st;
    const int64_t vs = vocab_end - vocab_start;
    if (ld_logits < vs || ld_logits > kMaxLogitsLd) return VP_ERR_SHAPE;
    if (ld_logits % 4 != 0) return VP_ERR_ALIGN;
    if (n == 0) return VP_OK;
    if (!hidden || !w_shard || !logits) return VP_ERR_NULL;
    if (!aligned(hidden, 16) || !aligned(w_shard, 16) || !aligned(logits, 16)) return VP_ERR_ALIGN;
    return hip_status(vp::launch_lmhead_logits(hidden, w_shard, n, h, vs, logits, ld_logits, stream));
}

int vp_logits_ce_stats(const float *logits, int64_t ld_logits, const int64_t *targets, int64_t n,
                       int64_t vocab_start, int64_t vocab_end, const float *m_ref, float *m_local,
                       float *s_local, float *zy_local, hipStream_t stream) {
    if (n < 0 || n > (1 << 20)) return VP_ERR_SHAPE;
    if (vocab_start < 0 || vocab_end <= vocab_start) return VP_ERR_RANGE;
    const int64_t vs = vocab_end - vocab_start;
    if (vs > (1 << 20) || ld_logits < vs || ld_logits > kMaxLogitsLd) return VP_ERR_SHAPE;
    if (ld_logits % 4 != 0) return VP_ERR_ALIGN;
    if (n == 0) return VP_OK;
    if (!logits || !targets || !m_local || !s_local || !zy_local) return VP_ERR_NULL;
    if (!aligned(logits, 16) || !aligned(targets, 8) || !aligned(m_local, 4) ||
        !aligned(s_local, 4) || !aligned(zy_local, 4) || (m_ref && !aligned(m_ref, 4)))
        return VP_ERR_ALIGN;
    return hip_status(vp::launch_logits_stats(logits, ld_logits, targets, n, vocab_start, vs, m_ref,
                                              m_local, s_local, zy_local, stream));
}

int vp_ce_max(const float *m, int64_t n, int32_t T, float *m_max, hipStream_t stream) {
    if (n < 0 || T < 1 || n > ((int64_t)1 << 31)) return VP_ERR_SHAPE;
    if (n == 0) return VP_OK;
    if (!m || !m_max) return VP_ERR_NULL;
    if (!aligned(m, 4) || !aligned(m_max, 4)) return VP_ERR_ALIGN;
    return hip_status(vp::launch_rows_max(m, n, T, m_max, stream));
}

int vp_logits_ce_bwd(const float *logits, int64_t ld_logits, const uint16_t *hidden,
                     const uint16_t *w_shard, const int64_t *targets, const float *lse, int64_t n,
                     int64_t h, int64_t vocab_start, int64_t vocab_end, int64_t ignore_index,
                     float grad_scale, float *dx, float *dw, void *workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    int st = check_shard(n, h, vocab_start, vocab_end);
    if (st != VP_OK) return st;
    const int64_t vs = vocab_end - vocab_start;
    if (ld_logits < vs || ld_logits > kMaxLogitsLd) return VP_ERR_SHAPE;
    if (ld_logits % 4 != 0) return VP_ERR_ALIGN;
    if (!dw) return VP_ERR_NULL;
    if (!aligned(dw, 16)) return VP_ERR_ALIGN;
    if (n > 0) {
        if (!logits || !hidden || !w_shard || !targets || !lse || !dx) return VP_ERR_NULL;
        if (!aligned(logits, 16) || !aligned(hidden, 16) || !aligned(w_shard, 16) ||
            !aligned(targets, 8) || !aligned(lse, 4) || !aligned(dx, 16))
            return VP_ERR_ALIGN;
        if (!workspace || !aligned(workspace, 256) ||
            workspace_bytes < vp::bwd_workspace(n, h, vs).bytes)
            return VP_ERR_WORKSPACE;
    }
    return hip_status(vp::launch_logits_ce_bwd(logits, ld_logits, hidden, w_shard, targets, lse, n, h,
                                               vocab_start, vs, ignore_index, grad_scale, dx, dw,
                                               workspace, stream));
}

}  // extern "C"
