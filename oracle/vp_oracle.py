"""Plain fp64 CPU oracle for the vocab-parallel embedding, LM head and cross entropy.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this module.  It shares no code with the HIP
library (no kernels, headers, helpers or constants): it only receives the same
input bits, widened exactly from bf16 to fp64 by the caller.

Everything here is the *definition* of what the fast path computes, written
out with NumPy in fp64; ``np.matmul`` is the only library routine used for the
contractions.  There is no blocking or fusion beyond splitting the token axis
into chunks to bound host memory, which changes no result.

Sources (the pages this method is described on):

* MiniMind-Tron, "5 Vocab Parallelism" -- section 5.1 (shard interval and the
  divisibility rule), 5.2.1 (masked embedding lookup and the V=8, T=2 worked
  example), 5.2.2 (LM head as a column-parallel linear), 5.3.1 (the stable
  cross-entropy decomposition and the three per-token statistics), 5.3.2
  (gradient p - onehot, subtracting only on the owning shard), 5.3.3
  (ignore_index and the mean over valid tokens).
* Interview note "Vocab parallelism" -- Figure 1 (id 5 with V=8, t=2),
  Figure 2 and the key-formula block (loss = log S - (z_y - m), the merge of
  per-shard max / sum-exp / target logit), the backward remark (softmax minus
  onehot, column-parallel rule for dX).
* Glossary "Tensor Parallelism" -- column-parallel linear: each shard's input
  gradient is a partial sum over shards.

Parity pins for every function live in ``tests/oracle_pins.py`` (run by
``tests/test_oracle.py``; ``tests/test_oracle_mutations.py`` checks that they
catch planted mistakes).
"""
from __future__ import annotations

import numpy as np

DEFAULT_IGNORE_INDEX = -100

__all__ = [
    "DEFAULT_IGNORE_INDEX", "shard_range", "padded_vocab", "embed_shard", "embed_shard_grad",
    "embed_shard_grad_rows", "logits",
    "shard_stats", "shard_sumexp", "combine_triples", "pages_sharded_ce", "dense_ce",
    "dense_dlogits", "shard_grads", "mean_scale", "lse_dense_chunked",
    "shard_stats_chunked", "dz_rows", "dz_cols", "shard_grads_chunked",
]


# ---------------------------------------------------------------------------
# shard bounds and the embedding lookup
# ---------------------------------------------------------------------------
def shard_range(V: int, T: int, t: int):
    """Vocabulary interval owned by shard t of T.

    "5 Vocab Parallelism", 5.1 / 5.2.1: shard t owns [t V/T, (t+1) V/T), and
    the vocabulary must split evenly (V % T == 0).
    """
    if T < 1 or not (0 <= t < T):
        raise ValueError(f"bad shard index t={t} for T={T}")
    if V % T != 0:
        raise ValueError(f"V={V} is not divisible by T={T}")
    vs = V // T
    return t * vs, (t + 1) * vs


def padded_vocab(V: int, T: int, multiple: int = 128) -> int:
    """Vocabulary size after padding so that every shard's V/T rows are a multiple of
    ``multiple``: the smallest V_pad >= V divisible by multiple * T (interview note
    "Vocab parallelism", the padding question: GPT-2's 50257 becomes 51200 for 8 ranks).
    The extra rows are ordinary rows of the table that no id or target uses; the method
    then runs unchanged on V_pad (5.1 holds since T divides V_pad)."""
    if V <= 0 or T < 1 or multiple < 1:
        raise ValueError(f"bad padding request V={V} T={T} multiple={multiple}")
    q = multiple * T
    return -(-V // q) * q


def embed_shard(ids, w_shard: np.ndarray, start: int, end: int) -> np.ndarray:
    """One shard's masked lookup.

    "5 Vocab Parallelism", 5.2.1 (and Figure 1 of the interview note): a token
    whose id lies in [start, end) gets row id - start of the local weight;
    every other token gets the zero row.  Works on any dtype (an index copy),
    so bf16 bit patterns come back bit-for-bit.
    """
    ids = np.asarray(ids, dtype=np.int64)
    out = np.zeros((ids.shape[0], w_shard.shape[1]), dtype=w_shard.dtype)
    own = (ids >= start) & (ids < end)
    out[own] = w_shard[ids[own] - start]
    return out


def embed_shard_grad(ids, dout: np.ndarray, start: int, end: int) -> np.ndarray:
    """Gradient of one shard's masked lookup with respect to its weight rows.

    The lookup of "5 Vocab Parallelism", 5.2.1 is linear in the shard's weight:
    out = P W_r, where P[i, k] = 1 when token i's id is owned and id - start == k,
    else 0.  Its adjoint is dW_r = P^T dOut: every owned token adds its output
    gradient to row id - start, off-shard tokens add nothing, and repeated ids
    accumulate.  (The pages state the lookup, not this backward; it is the
    plain adjoint.)  Returns fp64 [end - start, H].
    """
    ids = np.asarray(ids, dtype=np.int64)
    g = np.asarray(dout, dtype=np.float64)
    out = np.zeros((end - start, g.shape[1]))
    own = (ids >= start) & (ids < end)
    np.add.at(out, ids[own] - start, g[own])
    return out


def embed_shard_grad_rows(ids, dout: np.ndarray, start: int, rows) -> np.ndarray:
    """Rows ``rows`` (local indices) of ``embed_shard_grad``, each the fp64 sum of
    the output gradients of the tokens whose id is start + row."""
    ids = np.asarray(ids, dtype=np.int64)
    g = np.asarray(dout)
    out = np.zeros((len(rows), g.shape[1]))
    for k, r in enumerate(rows):
        sel = np.nonzero(ids == start + int(r))[0]
        if sel.size:
            out[k] = g[sel].astype(np.float64).sum(axis=0)
    return out


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------
def logits(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """z = X W^T in fp64 ("5 Vocab Parallelism", 5.2.2: [*, H] x [V/T, H]^T)."""
    return np.matmul(np.asarray(x, dtype=np.float64), np.asarray(w, dtype=np.float64).T)


def _check_targets(targets: np.ndarray, V: int, ignore_index: int) -> np.ndarray:
    t = np.asarray(targets, dtype=np.int64)
    valid = t != ignore_index
    if np.any((t[valid] < 0) | (t[valid] >= V)):
        raise ValueError("targets must lie in [0, V) or equal ignore_index")
    return valid


def shard_stats(z_shard: np.ndarray, targets, start: int):
    """Per-token statistics of one shard's logits.

    Returns (m_r, s_r, zy_r): the shard's own maximum, the sum of
    exp(z - m_r) over the shard, and the target logit when the target id lies
    in this shard (0 otherwise).  These are the three quantities of
    "5 Vocab Parallelism", 5.3.1 and Figure 2 of the interview note, with the
    sum taken about the shard's own maximum; ``combine_triples`` re-expresses
    it about the global maximum.
    """
    z = np.asarray(z_shard, dtype=np.float64)
    n, vs = z.shape
    t = np.asarray(targets, dtype=np.int64)
    m = z.max(axis=1)
    s = np.exp(z - m[:, None]).sum(axis=1)
    own = (t >= start) & (t < start + vs)
    zy = np.zeros(n, dtype=np.float64)
    rows = np.nonzero(own)[0]
    zy[rows] = z[rows, t[rows] - start]
    return m, s, zy


def shard_sumexp(z_shard: np.ndarray, m_ref) -> np.ndarray:
    """The second pass of the pages' order ("5 Vocab Parallelism", 5.3.1): one shard's
    sum of exp(z - m) about a given per-token maximum m (the global one, after the
    all-reduce MAX)."""
    z = np.asarray(z_shard, dtype=np.float64)
    return np.exp(z - np.asarray(m_ref, dtype=np.float64)[:, None]).sum(axis=1)


def combine_triples(m, s, zy, targets, ignore_index: int = DEFAULT_IGNORE_INDEX):
    """Merge T per-shard triples into the per-token loss.

    Global max M = max_r m_r; the global sum about M is
    S = sum_r s_r exp(m_r - M) (each shard's sum moved from its own maximum to
    M); the target logit z_y = sum_r zy_r (only the owner is non-zero).  Then
    loss = log S - (z_y - M) (interview note, key formulas; "5 Vocab
    Parallelism", 5.3.1), 0 at ignored tokens, and the mean over valid tokens
    divides by max(1, N_valid) (5.3.3).  Also returns lse = M + log S.
    """
    m = np.asarray(m, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    zy = np.asarray(zy, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    M = m.max(axis=0)
    S = (s * np.exp(m - M[None, :])).sum(axis=0)
    Zy = zy.sum(axis=0)
    lse = M + np.log(S)
    valid = t != ignore_index
    loss = np.where(valid, np.log(S) - (Zy - M), 0.0)
    mean = loss[valid].sum() / max(1, int(valid.sum()))
    return loss, lse, mean


def pages_sharded_ce(z_shards, targets, starts, ignore_index: int = DEFAULT_IGNORE_INDEX):
    """Cross entropy from per-shard logits in the order the pages give.

    "5 Vocab Parallelism", 5.3.1: first the global maximum of all shards' local
    maxima; then each shard's sum of exp(z - m) about that *global* maximum,
    summed over shards; the target logit taken on its owner and summed.
    Returns (loss, lse, mean).
    """
    t = np.asarray(targets, dtype=np.int64)
    zs = [np.asarray(z, dtype=np.float64) for z in z_shards]
    m = np.max(np.stack([z.max(axis=1) for z in zs]), axis=0)
    S = np.zeros_like(m)
    for z in zs:
        S += np.exp(z - m[:, None]).sum(axis=1)
    zy = np.zeros_like(m)
    for z, lo in zip(zs, starts):
        own = (t >= lo) & (t < lo + z.shape[1])
        rows = np.nonzero(own)[0]
        zy[rows] += z[rows, t[rows] - lo]
    valid = t != ignore_index
    loss = np.where(valid, np.log(S) - (zy - m), 0.0)
    mean = loss[valid].sum() / max(1, int(valid.sum()))
    return loss, m + np.log(S), mean


def dense_ce(z: np.ndarray, targets, ignore_index: int = DEFAULT_IGNORE_INDEX):
    """Textbook cross entropy over the full vocabulary.

    loss_n = -z[n, y_n] + M_n + log sum_j exp(z[n, j] - M_n), M_n = max_j z[n, j]
    ("5 Vocab Parallelism", 5.3.1), 0 where y_n == ignore_index, mean over
    valid tokens with max(1, N_valid) (5.3.3).  Returns (loss, lse, mean).
    """
    z = np.asarray(z, dtype=np.float64)
    valid = _check_targets(targets, z.shape[1], ignore_index)
    t = np.asarray(targets, dtype=np.int64)
    M = z.max(axis=1)
    lse = M + np.log(np.exp(z - M[:, None]).sum(axis=1))
    rows = np.nonzero(valid)[0]
    loss = np.zeros(z.shape[0], dtype=np.float64)
    loss[rows] = lse[rows] - z[rows, t[rows]]
    mean = loss[valid].sum() / max(1, int(valid.sum()))
    return loss, lse, mean


def mean_scale(targets, ignore_index: int = DEFAULT_IGNORE_INDEX) -> float:
    """d(mean loss)/d(loss_n) for a valid token: 1 / max(1, N_valid) (5.3.3)."""
    t = np.asarray(targets, dtype=np.int64)
    return 1.0 / max(1, int((t != ignore_index).sum()))


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------
def dense_dlogits(z: np.ndarray, targets, ignore_index: int = DEFAULT_IGNORE_INDEX,
                  scale: float | None = None) -> np.ndarray:
    """Gradient of the mean loss with respect to the logits.

    d loss_n / d z[n, j] = softmax(z_n)_j - [j == y_n] ("5 Vocab Parallelism",
    5.3.2; interview note, backward), times the mean's factor
    1 / max(1, N_valid) on valid rows and 0 on ignored rows (5.3.3).
    ``scale`` overrides the factor (the loss of a subset of tokens).
    """
    z = np.asarray(z, dtype=np.float64)
    valid = _check_targets(targets, z.shape[1], ignore_index)
    t = np.asarray(targets, dtype=np.int64)
    g = mean_scale(t, ignore_index) if scale is None else float(scale)
    M = z.max(axis=1, keepdims=True)
    e = np.exp(z - M)
    p = e / e.sum(axis=1, keepdims=True)
    rows = np.nonzero(valid)[0]
    p[rows, t[rows]] -= 1.0
    p[~valid] = 0.0
    return p * g


def shard_grads(x: np.ndarray, w_shard: np.ndarray, dz_shard: np.ndarray):
    """Gradients of one vocab shard of the LM head from its slice of dlogits.

    z_r = X W_r^T, so dX_r = dz_r W_r (this shard's *partial* input gradient;
    the sum over shards is the column-parallel rule of the "Tensor
    Parallelism" glossary entry and of the interview note's backward remark)
    and dW_r = dz_r^T X (local to the shard).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_shard, dtype=np.float64)
    dz = np.asarray(dz_shard, dtype=np.float64)
    return np.matmul(dz, w), np.matmul(dz.T, x)


# ---------------------------------------------------------------------------
# the same definitions evaluated on slices, for workloads whose dense logits
# would not fit in host memory at once
# ---------------------------------------------------------------------------
def lse_dense_chunked(x: np.ndarray, w: np.ndarray, chunk: int = 512) -> np.ndarray:
    """log sum_j exp(z[n, j]) over all rows of ``w`` for every token, token-chunked."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    out = np.empty(x.shape[0], dtype=np.float64)
    for a in range(0, x.shape[0], chunk):
        z = np.matmul(x[a:a + chunk], w.T)
        M = z.max(axis=1)
        out[a:a + chunk] = M + np.log(np.exp(z - M[:, None]).sum(axis=1))
    return out


def shard_stats_chunked(x: np.ndarray, w_shard: np.ndarray, targets, start: int,
                        chunk: int = 512):
    """``shard_stats(logits(x, w_shard), targets, start)`` evaluated token-chunked."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_shard, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    n = x.shape[0]
    m, s, zy = (np.empty(n) for _ in range(3))
    for a in range(0, n, chunk):
        m[a:a + chunk], s[a:a + chunk], zy[a:a + chunk] = shard_stats(
            np.matmul(x[a:a + chunk], w.T), t[a:a + chunk], start)
    return m, s, zy


def dz_rows(x_rows: np.ndarray, w_shard: np.ndarray, targets_rows, lse_rows,
            start: int, scale: float, ignore_index: int = DEFAULT_IGNORE_INDEX) -> np.ndarray:
    """Rows of dlogits restricted to one shard, given each token's full-vocabulary lse.

    softmax(z)_j = exp(z_j - lse); dz = scale * (softmax - onehot) on valid
    tokens, 0 on ignored ones (5.3.2, 5.3.3), for the columns of shard
    [start, start + Vs).
    """
    z = logits(x_rows, w_shard)
    t = np.asarray(targets_rows, dtype=np.int64)
    p = np.exp(z - np.asarray(lse_rows, dtype=np.float64)[:, None])
    own = (t >= start) & (t < start + z.shape[1]) & (t != ignore_index)
    rows = np.nonzero(own)[0]
    p[rows, t[rows] - start] -= 1.0
    p[t == ignore_index] = 0.0
    return p * scale


def dz_cols(x: np.ndarray, w_rows: np.ndarray, vocab_ids, targets, lse,
            scale: float, ignore_index: int = DEFAULT_IGNORE_INDEX) -> np.ndarray:
    """Columns of dlogits for the given global vocabulary ids, over all tokens.

    Same definition as ``dz_rows``; returns [N, len(vocab_ids)].
    """
    z = logits(x, w_rows)
    t = np.asarray(targets, dtype=np.int64)
    p = np.exp(z - np.asarray(lse, dtype=np.float64)[:, None])
    ids = np.asarray(vocab_ids, dtype=np.int64)
    p -= (t[:, None] == ids[None, :]).astype(np.float64)
    p[t == ignore_index] = 0.0
    return p * scale


def shard_grads_chunked(x: np.ndarray, w_shard: np.ndarray, targets, lse, start: int,
                        scale: float, ignore_index: int = DEFAULT_IGNORE_INDEX,
                        chunk: int = 512):
    """``shard_grads`` of one shard over all tokens, with its dlogits formed token-chunked.

    For each chunk of tokens, ``dz_rows`` gives the shard's columns of dlogits from the
    tokens' full-vocabulary lse; that chunk's rows of dX_r = dz_r W_r are stored and its
    dz_r^T X is added into dW_r = sum over chunks (the column-parallel partial and the local
    weight gradient of the interview note's backward remark).  Chunking only bounds host
    memory; it changes no term of either sum.  Returns fp64 (dX_r [N, H], dW_r [Vs, H]).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_shard, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64)
    ls = np.asarray(lse, dtype=np.float64)
    n = x.shape[0]
    dx = np.empty((n, w.shape[1]))
    dw = np.zeros(w.shape)
    for a in range(0, n, chunk):
        dz = dz_rows(x[a:a + chunk], w, t[a:a + chunk], ls[a:a + chunk], start, scale,
                     ignore_index)
        dx[a:a + chunk] = np.matmul(dz, w)
        dw += np.matmul(dz.T, x[a:a + chunk])
    return dx, dw
