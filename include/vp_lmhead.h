/*
 * vp_lmhead.h -- C ABI of the MI355X (gfx950) vocab-parallel LM head + cross entropy.
 *
 * One vocabulary shard of a language model's tied embedding / LM-head weight,
 * W_r = rows [vocab_start, vocab_end) of the [V, H] table, is used for
 *   - the masked embedding lookup (vp_embed_fwd) and its weight gradient
 *     (vp_embed_bwd),
 *   - the LM-head GEMM fused with the cross-entropy statistics, which never
 *     writes the [n, V/T] logits to memory (vp_lmhead_ce_fwd),
 *   - the merge of the T shards' statistics into the loss (vp_ce_combine),
 *     which stands in for the three per-token all-reduces of the method,
 *   - the local backward: dlogits = softmax - onehot, then dX_r and dW_r
 *     (vp_lmhead_ce_bwd),
 *   - the vocabulary padding of the interview note (vp_padded_vocab), and a
 *     materialised-logits comparator that stores the shard's logits instead of
 *     fusing them (vp_lmhead_logits, vp_logits_ce_stats, vp_ce_max,
 *     vp_logits_ce_bwd; at the end of this header).
 * Method: MiniMind-Tron "5 Vocab Parallelism" (sections 5.1-5.3.3) and the
 * interview note "Vocab parallelism" (Figures 1-2, key formulas, backward,
 * padding).
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless the argument says "host".
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major, contiguous.
 *   - The caller owns every buffer, workspaces included; the library holds no
 *     device memory and no mutable global state.  Calls are asynchronous on
 *     `stream` (0 = the null stream) and never synchronise; device-side faults
 *     surface at the caller's next synchronisation.
 *   - Returns VP_OK (0) or a negative vp_status.  Arguments are validated on
 *     the host before anything is launched; on an error nothing is launched
 *     and no output is touched.  n == 0 is valid (see each call).
 *   - Alignment: bf16 and fp32 tensors must be 16-byte aligned and H must be a
 *     multiple of 8 (rows then start on 16-byte boundaries); int64 arrays must
 *     be 8-byte aligned.  Otherwise VP_ERR_ALIGN.
 *   - Data contract (not checked on the device): each target lies in [0, V)
 *     or equals ignore_index.  A target outside the shard contributes nothing
 *     on that shard.
 */
#ifndef VP_LMHEAD_H
#define VP_LMHEAD_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    VP_OK = 0,
    VP_ERR_NULL = -1,       /* a required pointer is null                      */
    VP_ERR_SHAPE = -2,      /* a size is negative / zero where it must not be, too large
                               (n, h or Vs above 2^20 in the CE calls), or V % T != 0 */
    VP_ERR_RANGE = -3,      /* vocab_end <= vocab_start, or t outside [0, T)    */
    VP_ERR_ALIGN = -4,      /* H % 8 != 0 or a pointer is misaligned           */
    VP_ERR_WORKSPACE = -5,  /* workspace pointer null or smaller than required */
    VP_ERR_HIP = -6,        /* the HIP runtime reported an error at launch     */
    VP_ERR_SCRATCH = -7     /* the call needs more scratch than the fixed device buffer of
                               the allocation-free entry point holds               */
} vp_status;

/* Human-readable name of a status code (static string, never null). */
const char *vp_status_string(int status);

/*
 * vp_shard_range -- vocabulary interval owned by shard t of T.
 * "5 Vocab Parallelism", 5.1 and 5.2.1: shard t owns [t V/T, (t+1) V/T) and
 * V must be divisible by T.
 *   V, T, t : host scalars; 1 <= T, 0 <= t < T, V > 0.
 *   start, end : host pointers receiving the interval.
 * Errors: VP_ERR_NULL, VP_ERR_SHAPE (V <= 0, T < 1, V % T != 0), VP_ERR_RANGE.
 */
int vp_shard_range(int64_t V, int32_t T, int32_t t, int64_t *start, int64_t *end);

/*
 * vp_padded_vocab -- vocabulary size after padding so that every shard's rows are a
 * multiple of `multiple` (the interview note "Vocab parallelism", padding question:
 * each rank's V/t a multiple of 128; GPT-2's 50257 becomes 51200 for 8 ranks):
 *   V_pad = the smallest multiple of multiple * T that is >= V.
 * The extra rows are ordinary rows of the (padded) table that no id or target uses;
 * every other entry point then runs unchanged with V_pad in place of V.
 *   V, T, multiple : host scalars, all >= 1.   V_pad : host pointer receiving the size.
 * Errors: VP_ERR_NULL, VP_ERR_SHAPE (V <= 0, T < 1, multiple < 1, or overflow).
 */
int vp_padded_vocab(int64_t V, int32_t T, int64_t multiple, int64_t *V_pad);

/*
 * vp_embed_fwd -- masked vocab-parallel embedding lookup of one shard.
 * "5 Vocab Parallelism", 5.2.1; interview note, Figure 1:
 *   out[i, :] = w_shard[ids[i] - vocab_start, :]  if vocab_start <= ids[i] < vocab_end
 *   out[i, :] = +0.0                              otherwise (any int64 id, negative included)
 * Summing the T shards' outputs gives the dense lookup (the all-reduce of the
 * method); this call produces one shard's term.  The result is a bit copy.
 *   ids      int64 [n]
 *   w_shard  bf16  [vocab_end - vocab_start, h]  (the tied LM-head shard)
 *   out      bf16  [n, h], overwritten
 * n == 0: no-op.  Errors: NULL, SHAPE (n < 0, h <= 0), RANGE, ALIGN, HIP.
 */
int vp_embed_fwd(const int64_t *ids, int64_t n,
                 const uint16_t *w_shard, int64_t vocab_start, int64_t vocab_end, int64_t h,
                 uint16_t *out, hipStream_t stream);

/* Bytes of device workspace vp_embed_bwd needs (0 when n == 0 or the sizes are invalid). Host-only. */
size_t vp_embed_bwd_workspace(int64_t n, int64_t h, int64_t vocab_start, int64_t vocab_end);

/*
 * vp_embed_bwd -- weight gradient of one shard's masked lookup: the adjoint of
 * vp_embed_fwd.  "5 Vocab Parallelism", 5.2.1 defines the lookup, which is linear
 * in the shard's rows; its gradient scatters the output gradient back:
 *   dw[ids[i] - vocab_start, :] += dout[i, :]   for every i with vocab_start <= ids[i] < vocab_end
 * Repeated ids accumulate; tokens whose id lies outside the shard (any int64,
 * negative included) add nothing; rows that no owned id names are left unchanged.
 * The result is ADDED to dw, so the tied shard's LM-head gradient (vp_lmhead_ce_bwd's
 * dw) can be passed in.  Deterministic: each row's tokens are summed in fp32 in a
 * fixed order (increasing token index within fixed blocks of the id-sorted tokens),
 * then added to dw once; no floating-point atomics.
 *   ids   int64 [n]
 *   dout  bf16  [n, h]   (gradient of vp_embed_fwd's output)
 *   dw    fp32  [vocab_end - vocab_start, h], read and written
 *   workspace >= vp_embed_bwd_workspace(...) bytes, 256-byte aligned, contents scratch
 * n == 0: no-op.  Errors: NULL, SHAPE (n < 0, n > 2^24, h <= 0, more than 2^31 - 1
 * rows), RANGE, ALIGN, WORKSPACE, HIP.
 */
int vp_embed_bwd(const int64_t *ids, int64_t n, const uint16_t *dout,
                 int64_t vocab_start, int64_t vocab_end, int64_t h, float *dw,
                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace vp_lmhead_ce_fwd needs (0 when n == 0). Host-only. */
size_t vp_lmhead_ce_fwd_workspace(int64_t n, int64_t h, int64_t vocab_start, int64_t vocab_end);

/*
 * vp_lmhead_ce_fwd -- LM-head GEMM of one shard fused with its cross-entropy
 * statistics ("5 Vocab Parallelism", 5.2.2 and 5.3.1; interview note,
 * Figure 2).  With z = hidden * w_shard^T (fp32 accumulation of bf16
 * products), for each token i over the shard's Vs = vocab_end - vocab_start
 * columns:
 *   m_local[i]  = max_j z[i, j]
 *   s_local[i]  = sum_j exp(z[i, j] - m_local[i])     (about the shard's own max)
 *   zy_local[i] = z[i, targets[i] - vocab_start] if the target is in the shard, else 0
 * The [n, Vs] logits never reach memory.
 *   hidden   bf16  [n, h];  w_shard bf16 [Vs, h];  targets int64 [n]
 *   m_local, s_local, zy_local  fp32 [n] each, overwritten (typically row t of [T, n] arrays)
 *   workspace >= vp_lmhead_ce_fwd_workspace(...) bytes, 256-byte aligned, contents scratch
 * n == 0: no-op.  Errors: NULL, SHAPE, RANGE, ALIGN, WORKSPACE, HIP.
 */
int vp_lmhead_ce_fwd(const uint16_t *hidden, const uint16_t *w_shard, const int64_t *targets,
                     int64_t n, int64_t h, int64_t vocab_start, int64_t vocab_end,
                     float *m_local, float *s_local, float *zy_local,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Size of the fixed device scratch buffer of vp_lmhead_ce_fwd_noalloc (64 MiB). */
#define VP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * vp_lmhead_ce_fwd_noalloc -- vp_lmhead_ce_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, bit for bit, with the workspace taken from a
 * fixed buffer of VP_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  Calls no allocator.  The caller still passes inputs and outputs
 * (arguments as vp_lmhead_ce_fwd, without the workspace).
 *   Limit: vp_lmhead_ce_fwd_workspace(n, h, vocab_start, vocab_end) must not exceed
 *   VP_NOALLOC_SCRATCH_BYTES (e.g. n = 16384 tokens with a 19008-row shard needs 29.3 MB),
 *   else VP_ERR_SCRATCH and nothing is launched.
 *   Every call on one GPU uses that GPU's one buffer: calls that overlap in time on one GPU
 *   (on different streams, or from different threads) race and must be serialised by the
 *   caller.  The buffer needs no clearing: every byte a call reads it has written first.
 *   The buffer of the stream's GPU is looked up on the first call on that GPU (the device
 *   is switched for that lookup and restored).
 * n == 0: no-op.  Errors: NULL, SHAPE, RANGE, ALIGN, SCRATCH, HIP.
 */
int vp_lmhead_ce_fwd_noalloc(const uint16_t *hidden, const uint16_t *w_shard,
                             const int64_t *targets, int64_t n, int64_t h,
                             int64_t vocab_start, int64_t vocab_end,
                             float *m_local, float *s_local, float *zy_local, hipStream_t stream);

/*
 * vp_ce_combine -- merge T shards' statistics into the loss; stands in for the
 * all-reduce MAX / SUM / SUM of "5 Vocab Parallelism", 5.3.1 (interview note,
 * Figure 2 and key formulas), with the mean of 5.3.3:
 *   M = max_r m[r, i];  S = sum_r s[r, i] * exp(m[r, i] - M);  Zy = sum_r zy[r, i]
 *   loss[i] = log S - (Zy - M)   (0 where targets[i] == ignore_index)
 *   lse[i]  = M + log S          (the full-vocabulary log-sum-exp, for the backward)
 *   loss_mean[0] = sum_i loss[i] / max(1, #{i : targets[i] != ignore_index})
 *   m, s, zy  fp32 [T, n] row-major (row r = shard r's vp_lmhead_ce_fwd output)
 *   targets   int64 [n];  loss, lse fp32 [n];  loss_mean fp32 [1]; all overwritten
 * n == 0: writes loss_mean = 0 only.  Errors: NULL, SHAPE (n < 0, n > 2^31, T < 1), ALIGN, HIP.
 */
int vp_ce_combine(const float *m, const float *s, const float *zy,
                  const int64_t *targets, int64_t n, int32_t T, int64_t ignore_index,
                  float *loss, float *lse, float *loss_mean, hipStream_t stream);

/* Bytes of device workspace vp_lmhead_ce_bwd needs. Host-only. */
size_t vp_lmhead_ce_bwd_workspace(int64_t n, int64_t h, int64_t vocab_start, int64_t vocab_end);

/*
 * vp_lmhead_ce_bwd -- local backward of one shard ("5 Vocab Parallelism",
 * 5.3.2-5.3.3; interview note, backward; glossary "Tensor Parallelism",
 * column-parallel input gradient).  Recomputes z = hidden * w_shard^T, then
 *   dz[i, j] = g_i * (exp(z[i, j] - lse[i]) - [j == targets[i] - vocab_start])
 *   g_i = grad_scale if targets[i] != ignore_index else 0
 *   dx = dz * w_shard   -- this shard's PARTIAL input gradient (sum over shards = dX)
 *   dw = dz^T * hidden  -- this shard's weight gradient
 * No inter-shard communication is needed.  dz is rounded to bf16 before the
 * two GEMMs (fp32 accumulation).
 *   lse        fp32 [n] from vp_ce_combine
 *   grad_scale host scalar: upstream gradient of each valid token's loss
 *              (1 / max(1, N_valid) for the mean loss)
 *   dx  fp32 [n, h], overwritten;  dw fp32 [Vs, h], overwritten (zeros when n == 0)
 *   workspace >= vp_lmhead_ce_bwd_workspace(...) bytes, 256-byte aligned, contents scratch
 * Errors: NULL, SHAPE, RANGE, ALIGN, WORKSPACE, HIP.
 */
int vp_lmhead_ce_bwd(const uint16_t *hidden, const uint16_t *w_shard, const int64_t *targets,
                     const float *lse, int64_t n, int64_t h,
                     int64_t vocab_start, int64_t vocab_end, int64_t ignore_index,
                     float grad_scale, float *dx, float *dw,
                     void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Materialised-logits comparator.  The same step with one shard's logits stored in HBM,
 * as the pages' tensor-parallel baseline holds them ([S, B, V/T] per rank, fp32).  Not the
 * fused hot path: it exists to measure the memory and time the fused path saves
 * ("5 Vocab Parallelism", 5.3.1-5.3.2).  Conventions as above; ld_logits is the row
 * stride of the [n, ld_logits] fp32 logits, a multiple of 4 with Vs <= ld_logits <= 2^20 + 1024.
 * ------------------------------------------------------------------------------------ */

/* logits[i, j] = (hidden w_shard^T)[i, j] for j < Vs, fp32 (columns Vs .. round_up(Vs, 4)
 * are written with zeros).  n == 0: no-op.  Errors: NULL, SHAPE, RANGE, ALIGN, HIP. */
int vp_lmhead_logits(const uint16_t *hidden, const uint16_t *w_shard, int64_t n, int64_t h,
                     int64_t vocab_start, int64_t vocab_end, float *logits, int64_t ld_logits,
                     hipStream_t stream);

/* Per-token statistics of one shard's stored logits (5.3.1):
 *   m_ref == NULL: m_local = max_j z, s_local = sum_j exp(z - m_local)  (one read);
 *   m_ref != NULL: m_local = m_ref, s_local = sum_j exp(z - m_ref)      (the pages' second
 *                  pass, m_ref = the global maximum from vp_ce_max);
 *   zy_local = z[targets - vocab_start] if the target lies in the shard, else 0.
 * The outputs feed vp_ce_combine unchanged.  n == 0: no-op.
 * Errors: NULL, SHAPE (n or Vs above 2^20), RANGE, ALIGN, HIP. */
int vp_logits_ce_stats(const float *logits, int64_t ld_logits, const int64_t *targets, int64_t n,
                       int64_t vocab_start, int64_t vocab_end, const float *m_ref,
                       float *m_local, float *s_local, float *zy_local, hipStream_t stream);

/* m_max[i] = max_r m[r, i] over the T rows of m [T, n] (the all-reduce MAX of 5.3.1 on one
 * GPU).  n == 0: no-op.  Errors: NULL, SHAPE, ALIGN, HIP. */
int vp_ce_max(const float *m, int64_t n, int32_t T, float *m_max, hipStream_t stream);

/* Backward from the stored logits (5.3.2): dz = g (exp(z - lse) - onehot) read from logits
 * instead of recomputed, then dx and dw exactly as vp_lmhead_ce_bwd (same arguments,
 * semantics and workspace: vp_lmhead_ce_bwd_workspace). */
int vp_logits_ce_bwd(const float *logits, int64_t ld_logits, const uint16_t *hidden,
                     const uint16_t *w_shard, const int64_t *targets, const float *lse, int64_t n,
                     int64_t h, int64_t vocab_start, int64_t vocab_end, int64_t ignore_index,
                     float grad_scale, float *dx, float *dw, void *workspace,
                     size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VP_LMHEAD_H */
