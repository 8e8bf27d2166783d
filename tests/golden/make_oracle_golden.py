"""Write the oracle's expected values for the full-size workloads.

    python tests/golden/make_oracle_golden.py [workload ...]

Calls only ``oracle/`` (fp64 NumPy) and the seeded input generators
(``vp_inputs``); nothing from the HIP path.  For each workload whose dense
logits are too large to recompute inside a GPU test (and for the small-LM workload,
whose bench timing is gated on it), it stores per token

  lse   the full-vocabulary log-sum-exp (fp64)
  loss  the per-token cross entropy (fp64)

in ``oracle_<workload>.npz`` next to this script.  The GPU tests regenerate
the same input bits from the same seeds and derive everything else they
compare (statistics of shard 0, sampled rows of dX and dW) from these values
with the oracle at test time.

``sweep`` writes ``oracle_sweep.npz`` for the benchmark's scaling sweep (shard 0 of
width 16032 at nine (N, H) shapes, the other seven shards given as fixed statistics):
per shape, every token's loss (fp64) and the oracle's dX and dW on the rows
``vp_inputs.sweep_samples`` names (stored as fp32; the gate's bar is relative 1e-2).
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import vp_inputs  # noqa: E402


def _f64(bits):
    return vp_inputs.bf16_bits_to_f64(bits)


def _dense_chunked(x, w, targets, chunk):
    """oracle.dense_ce over the full vocabulary, one chunk of tokens at a time."""
    n = x.shape[0]
    lse, loss = np.empty(n), np.empty(n)
    for a in range(0, n, chunk):
        loss[a:a + chunk], lse[a:a + chunk], _ = oracle.dense_ce(
            oracle.logits(x[a:a + chunk], w), targets[a:a + chunk])
    valid = targets != oracle.DEFAULT_IGNORE_INDEX
    return {"lse": lse, "loss": loss, "mean": np.array(loss[valid].sum() / max(1, int(valid.sum())))}


def golden_shard_8b():
    """Dense cross entropy over all V = 128256 rows (all eight shards materialised)."""
    inp = vp_inputs.make_inputs("shard_8b")
    return _dense_chunked(_f64(inp.x), _f64(inp.w), inp.targets, chunk=512)


def golden_large_vocab():
    """Shard 0 computed from data, shards 1..7 from the synthetic statistics."""
    inp = vp_inputs.make_inputs("large_vocab")
    m, s, zy = vp_inputs.synthetic_triples("large_vocab", inp.targets)
    m0, s0, zy0 = oracle.shard_stats_chunked(_f64(inp.x), _f64(inp.w), inp.targets, 0, chunk=512)
    M = m.astype(np.float64)
    S = s.astype(np.float64)
    Z = zy.astype(np.float64)
    M[0], S[0], Z[0] = m0, s0, zy0
    loss, lse, mean = oracle.combine_triples(M, S, Z, inp.targets)
    return {"lse": lse, "loss": loss, "mean": np.array(mean)}


def golden_embedding_heavy():
    """T = 1 cross entropy over the full V = 256000 on N = 4096 tokens."""
    inp = vp_inputs.make_inputs("embedding_heavy")
    return _dense_chunked(_f64(inp.x), _f64(inp.w), inp.targets, chunk=256)


def golden_small_lm():
    """Dense cross entropy over V = 6400 (both shards) on N = 4096 tokens."""
    inp = vp_inputs.make_inputs("small_lm")
    return _dense_chunked(_f64(inp.x), _f64(inp.w), inp.targets, chunk=1024)


def golden_sweep(Vs=16032, T=8):
    out = {}
    for N, H in vp_inputs.SWEEP_SHAPES:
        xb, wb, y = vp_inputs.sweep_inputs(N, H, Vs, T)
        x, w = _f64(xb), _f64(wb)
        m0, s0, zy0 = oracle.shard_stats_chunked(x, w, y, 0, chunk=1024)
        ones = np.ones(N)
        loss, lse, _ = oracle.combine_triples(
            np.stack([m0] + [ones] * (T - 1)), np.stack([s0] + [1000.0 * ones] * (T - 1)),
            np.stack([zy0] + [0.0 * ones] * (T - 1)), y)
        g = 1.0 / N
        rows, cols = vp_inputs.sweep_samples(N, H, y, Vs)
        key = f"{N}x{H}"
        out[f"{key}_loss"] = loss
        out[f"{key}_dx"] = (oracle.dz_rows(x[rows], w, y[rows], lse[rows], 0, g) @ w).astype(np.float32)
        out[f"{key}_dw"] = (oracle.dz_cols(x, w[cols], cols, y, lse, g).T @ x).astype(np.float32)
        print(f"  sweep {key} done", flush=True)
    out["mean"] = np.array(0.0)   # (no single mean: one loss vector per shape)
    return out


MAKERS = {"shard_8b": golden_shard_8b, "large_vocab": golden_large_vocab,
          "embedding_heavy": golden_embedding_heavy, "small_lm": golden_small_lm,
          "sweep": golden_sweep}


def main(names):
    for name in names or [k for k in MAKERS if k != "sweep"]:
        t = time.time()
        out = MAKERS[name]()
        path = os.path.join(HERE, f"oracle_{name}.npz")
        np.savez_compressed(path, **out)
        print(f"{name}: wrote {path} in {time.time() - t:.1f}s  mean loss {float(out['mean']):.6f}",
              flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
