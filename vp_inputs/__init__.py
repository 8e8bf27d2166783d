"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module only *makes data*: bf16 bit patterns, token ids, targets and the
synthetic per-shard triples of the large-vocab workload.  It contains none of
the method's arithmetic (no logits, no soft-max, no gradients), so that the
oracle under ``oracle/`` and the HIP library never share code, only inputs.

Every array is produced by NumPy's PCG64 ``Generator`` from a fixed seed, so the
same bits come out on every machine.  Floating-point inputs are drawn in fp32,
scaled, then rounded to bf16 with round-to-nearest-even and returned as
``uint16`` bit patterns; both sides widen those same bits.

Workloads (sizes and distributions as the five workload descriptions give
them; where those leave a detail open, the choice is stated beside it):

* ``tiny``              N=6, H=32, V=16, T=4, logits std ~5; plus the V=8, T=2
                        embedding example with ids [1, 6].
* ``small_lm``          N=4096 (B=8, S=512), H=512, V=6400, T=2.
* ``shard_8b``          N=8192, H=4096, V=128256, T=8 (shard [16032, 4096]),
                        Zipf(1.1) targets.
* ``large_vocab``       N=16384, H=8192, V=152064, T=8 (shard [19008, 8192]),
                        uniform targets, 7 synthetic per-shard triples.
* ``embedding_heavy``   embedding V=256000, H=4096, T=4, N=65536 Zipf(1.0) ids;
                        then a T=1 cross entropy on N=4096 tokens.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Dict, Optional

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "bf16_bits_to_f64",
    "zipf_ids", "Workload", "WORKLOADS", "make_inputs", "Inputs",
    "synthetic_triples", "SWEEP_SHAPES", "sweep_inputs",
]


# ----------------------------------------------------------------------------
# bf16 bit handling
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(a) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even) -> uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns to fp64 (exact)."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def _normal_bf16(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    """N(0, scale^2) drawn in fp32 and rounded to bf16 bits."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    # round to nearest even in place (the fp32 buffer is scratch here)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    u += ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = (u >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


# ----------------------------------------------------------------------------
# Zipf ids over a finite vocabulary
# ----------------------------------------------------------------------------
def zipf_ids(rng: np.random.Generator, n: int, V: int, s: float,
             perm: np.ndarray) -> np.ndarray:
    """``n`` ids with P(rank k) proportional to k**-s for k = 1..V.

    Sampled by inverse CDF over the finite support (s = 1.0 is allowed), then
    rank k is sent to id ``perm[k-1]`` so that frequent ids are spread over the
    whole vocabulary instead of all landing on the first shard.
    """
    k = np.arange(1, V + 1, dtype=np.float64)
    cdf = np.cumsum(k ** (-float(s)))
    cdf /= cdf[-1]
    u = rng.random(n)
    rank = np.minimum(np.searchsorted(cdf, u, side="right"), V - 1)
    return perm[rank].astype(np.int64)


# ----------------------------------------------------------------------------
# Workload table
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    N: int            # tokens for the cross entropy
    H: int            # hidden size
    V: int            # full vocabulary of the cross entropy
    T: int            # number of vocab shards
    x_scale: float    # std of hidden
    w_scale: float    # std of the weight
    targets: str      # "uniform" | "zipf"
    zipf_s: float = 0.0
    # embedding lookup riding alongside (tied weight unless stated)
    embed_V: int = 0
    embed_T: int = 0
    embed_N: int = 0
    embed_H: int = 0
    embed_ids: str = ""          # "uniform" | "zipf" | "fixed"
    synthetic_other_shards: bool = False   # large_vocab: shards 1..T-1 given as triples
    only_shard0_weight: bool = False       # only W_0 is materialised

    @property
    def Vs(self) -> int:
        return self.V // self.T


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", seed=0, N=6, H=32, V=16, T=4,
                     x_scale=1.0, w_scale=5.0 / math.sqrt(32.0), targets="uniform",
                     embed_V=8, embed_T=2, embed_N=2, embed_H=32, embed_ids="fixed"),
    "small_lm": Workload("small_lm", seed=1, N=4096, H=512, V=6400, T=2,
                         x_scale=1.0, w_scale=0.02, targets="uniform",
                         embed_V=6400, embed_T=2, embed_N=4096, embed_H=512,
                         embed_ids="uniform"),
    "shard_8b": Workload("shard_8b", seed=2, N=8192, H=4096, V=128256, T=8,
                         x_scale=1.0, w_scale=0.02, targets="zipf", zipf_s=1.1,
                         embed_V=128256, embed_T=8, embed_N=8192, embed_H=4096,
                         embed_ids="zipf"),
    "large_vocab": Workload("large_vocab", seed=3, N=16384, H=8192, V=152064, T=8,
                            x_scale=1.0, w_scale=0.01, targets="uniform",
                            synthetic_other_shards=True, only_shard0_weight=True),
    "embedding_heavy": Workload("embedding_heavy", seed=4, N=4096, H=4096, V=256000, T=1,
                                x_scale=1.0, w_scale=0.02, targets="zipf", zipf_s=1.0,
                                embed_V=256000, embed_T=4, embed_N=65536, embed_H=4096,
                                embed_ids="zipf"),
}

# child-stream indices of the SeedSequence of a workload
_S_X, _S_TGT, _S_IDS, _S_PERM, _S_TRIPLES, _S_EMBW = 0, 1, 2, 3, 4, 5
_S_W0 = 8   # spawn-key prefix of the weight row blocks
_S_DOUT0 = 9   # spawn-key prefix of the lookup's output-gradient row blocks
_N_CHILD = 8


@dataclasses.dataclass
class Inputs:
    wl: Workload
    x: Optional[np.ndarray]            # uint16 [N, H]
    w: Optional[np.ndarray]            # uint16 [V, H] (or [Vs, H] when only shard 0)
    targets: Optional[np.ndarray]      # int64 [N]
    ids: Optional[np.ndarray]          # int64 [embed_N]
    embed_w: Optional[np.ndarray]      # uint16 weight used by the lookup
    embed_w_rows: int                  # rows of embed_w that exist (V or Vs)

    def w_shard(self, r: int) -> np.ndarray:
        vs = self.wl.Vs
        if self.wl.only_shard0_weight:
            assert r == 0, "only shard 0 is materialised for this workload"
            return self.w
        return self.w[r * vs:(r + 1) * vs]


def _children(seed: int):
    return np.random.SeedSequence(seed).spawn(_N_CHILD)


def _perm(ch, V: int) -> np.ndarray:
    return np.random.Generator(np.random.PCG64(ch[_S_PERM])).permutation(V)


_ROW_BLOCK = 1024   # the full weight is drawn in independent blocks of rows


def make_weight_rows(wl: Workload, start: int, end: int) -> np.ndarray:
    """Rows [start, end) of the full [V, H] weight (bf16 bits).

    Row block b (rows [b*1024, (b+1)*1024)) always comes from its own PCG64
    stream, so any range -- one shard, or the whole vocabulary -- is produced
    with the same bits without materialising the rest.
    """
    assert 0 <= start <= end <= wl.V
    out = np.empty((end - start, wl.H), dtype=np.uint16)
    b0, b1 = start // _ROW_BLOCK, (end + _ROW_BLOCK - 1) // _ROW_BLOCK

    def one_block(b: int) -> None:
        lo, hi = b * _ROW_BLOCK, min((b + 1) * _ROW_BLOCK, wl.V)
        ss = np.random.SeedSequence(entropy=wl.seed, spawn_key=(_S_W0, b))
        blk = _normal_bf16(np.random.Generator(np.random.PCG64(ss)), (hi - lo, wl.H),
                           wl.w_scale)
        a, z = max(lo, start), min(hi, end)
        out[a - start:z - start] = blk[a - lo:z - lo]

    # blocks are independent streams, so threads change nothing in the result
    workers = max(1, min(16, len(os.sched_getaffinity(0)), b1 - b0))
    if workers == 1:
        for b in range(b0, b1):
            one_block(b)
    else:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one_block, range(b0, b1)))
    return out


def make_embed_output_grad(name: str, scale: float = 1.0) -> np.ndarray:
    """Gradient of the lookup's output, [embed_N, embed_H] bf16 bits ~ N(0, scale^2),
    drawn in independent 1024-row blocks (like the weight) so it can be made in parallel."""
    wl = WORKLOADS[name]
    n, h = wl.embed_N, wl.embed_H
    out = np.empty((n, h), dtype=np.uint16)

    def one_block(b: int) -> None:
        lo, hi = b * _ROW_BLOCK, min((b + 1) * _ROW_BLOCK, n)
        ss = np.random.SeedSequence(entropy=wl.seed, spawn_key=(_S_DOUT0, b))
        out[lo:hi] = _normal_bf16(np.random.Generator(np.random.PCG64(ss)), (hi - lo, h), scale)

    nb = (n + _ROW_BLOCK - 1) // _ROW_BLOCK
    workers = max(1, min(16, len(os.sched_getaffinity(0)), nb))
    if workers == 1:
        for b in range(nb):
            one_block(b)
    else:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(one_block, range(nb)))
    return out


def make_weight_shard(wl: Workload, r: int) -> np.ndarray:
    """Rows [r*Vs, (r+1)*Vs) of the LM-head / tied embedding weight (bf16 bits)."""
    return make_weight_rows(wl, r * wl.Vs, (r + 1) * wl.Vs)


def make_inputs(name: str, *, with_weight: bool = True, shards=None) -> Inputs:
    """Generate every input array of a workload.

    ``shards`` restricts which weight shards are materialised (the rest of
    ``w`` is then left as zeros); by default all of them are (only shard 0 for
    ``large_vocab``).
    """
    wl = WORKLOADS[name]
    ch = _children(wl.seed)
    g = lambda i: np.random.Generator(np.random.PCG64(ch[i]))
    x = _normal_bf16(g(_S_X), (wl.N, wl.H), wl.x_scale)

    perm = _perm(ch, wl.V)
    if wl.targets == "uniform":
        targets = g(_S_TGT).integers(0, wl.V, wl.N, dtype=np.int64)
    else:
        targets = zipf_ids(g(_S_TGT), wl.N, wl.V, wl.zipf_s, perm)

    w = None
    if with_weight:
        if wl.only_shard0_weight:
            w = make_weight_shard(wl, 0)
        else:
            w = np.zeros((wl.V, wl.H), dtype=np.uint16)
            rs = range(wl.T) if shards is None else shards
            for r in rs:
                w[r * wl.Vs:(r + 1) * wl.Vs] = make_weight_shard(wl, r)

    ids = None
    embed_w = None
    rows = 0
    if wl.embed_N:
        if wl.embed_ids == "fixed":
            # the worked lookup example: V=8 split over two ranks, ids [1, 6]
            ids = np.array([1, 6], dtype=np.int64)
            embed_w = _normal_bf16(g(_S_EMBW), (wl.embed_V, wl.embed_H), 1.0)
            rows = wl.embed_V
        else:
            if wl.embed_ids == "uniform":
                ids = g(_S_IDS).integers(0, wl.embed_V, wl.embed_N, dtype=np.int64)
            else:
                assert wl.embed_V == wl.V
                ids = zipf_ids(g(_S_IDS), wl.embed_N, wl.embed_V, wl.zipf_s, perm)
            # tied weight: the lookup reads the same [V, H] tensor as the LM head
            embed_w = w
            rows = 0 if w is None else w.shape[0]
    return Inputs(wl=wl, x=x, w=w, targets=targets, ids=ids, embed_w=embed_w,
                  embed_w_rows=rows)


def synthetic_triples(name: str, targets: np.ndarray):
    """Per-shard (m_r, s_r, zy_r) for shards r = 1..T-1 of ``large_vocab``.

    Only the statistics the cross entropy exchanges between shards are made up
    here; shard 0 is always computed from real data.  Valid by construction:
    m_r finite, 1 <= s_r <= Vs, and zy_r = m_r - U(0, 4) on the shard that owns
    the target, 0 elsewhere.  Returns float32 arrays of shape [T, N] whose row
    0 is left as NaN (to be filled by the caller).
    """
    wl = WORKLOADS[name]
    ch = _children(wl.seed)
    g = np.random.Generator(np.random.PCG64(ch[_S_TRIPLES]))
    T, N, Vs = wl.T, wl.N, wl.Vs
    m = np.full((T, N), np.nan, dtype=np.float32)
    s = np.full((T, N), np.nan, dtype=np.float32)
    zy = np.full((T, N), np.nan, dtype=np.float32)
    mbar = 3.6
    m[1:] = (mbar + 0.3 * g.standard_normal((T - 1, N))).astype(np.float32)
    s[1:] = g.uniform(500.0, 1100.0, (T - 1, N)).astype(np.float32)
    gap = g.uniform(0.0, 4.0, (T - 1, N)).astype(np.float32)
    owner = np.asarray(targets) // Vs
    zy[1:] = 0.0
    for r in range(1, T):
        own = owner == r
        zy[r, own] = m[r, own] - gap[r - 1, own]
    return m, s, zy


# ----------------------------------------------------------------------------
# the benchmark's scaling sweep at the 8B-class shard width
# ----------------------------------------------------------------------------
SWEEP_SHAPES = [(1024, 4096), (2048, 4096), (4096, 4096), (8192, 4096), (16384, 4096),
                (32768, 4096), (8192, 1024), (8192, 2048), (8192, 8192)]


def sweep_inputs(N: int, H: int, Vs: int = 16032, T: int = 8):
    """Inputs of one scaling-sweep shape: X ~ N(0, 1) [N, H] and shard 0's W ~ N(0, 0.02)
    [Vs, H], both rounded to bf16 bits, and targets uniform over the T Vs ids, from one
    PCG64 generator seeded N * 7 + H (X first, then W, then the targets).  The other shards
    enter only through fixed statistics (m = 1, s = 1000, target logit 0)."""
    rng = np.random.default_rng(N * 7 + H)
    x = f32_to_bf16_bits(rng.standard_normal((N, H), dtype=np.float32))
    w = f32_to_bf16_bits(np.float32(0.02) * rng.standard_normal((Vs, H), dtype=np.float32))
    y = rng.integers(0, Vs * T, N).astype(np.int64)
    return x, w, y


def sweep_samples(N: int, H: int, y: np.ndarray, Vs: int = 16032):
    """The rows the sweep's gate compares: 4 token rows of dX and 6 vocabulary rows of dW
    (4 random ids and the first 2 owned targets), seeded by the shape."""
    rows = np.sort(np.random.default_rng(N).choice(N, 4, replace=False))
    own = y[y < Vs]
    cols = np.unique(np.concatenate([np.random.default_rng(H).choice(Vs, 4, replace=False),
                                     own[:2]])).astype(np.int64)
    return rows, cols
