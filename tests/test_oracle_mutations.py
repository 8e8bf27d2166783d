"""Plant plausible mistakes in a copy of the oracle and check that a pin catches each.

Every mutation is a small source edit (a dropped term, a wrong sign, a wrong
index or a transposed operand) applied to the oracle's text; the edited copy
is loaded as a fresh module on the CPU, and at least one pin must fail on it.
"""
import inspect
import types

import pytest

import oracle.vp_oracle as vp_oracle
from oracle_pins import ALL_PINS

MUTATIONS = [
    # combine: drop the move of each shard's sum to the global maximum
    ("S = (s * np.exp(m - M[None, :])).sum(axis=0)", "S = s.sum(axis=0)"),
    # combine: wrong sign of the target logit
    ("loss = np.where(valid, np.log(S) - (Zy - M), 0.0)", "loss = np.where(valid, np.log(S) + (Zy - M), 0.0)"),
    # combine: mean over all tokens instead of valid ones
    ("mean = loss[valid].sum() / max(1, int(valid.sum()))\n    return loss, lse, mean\n\n\ndef pages",
     "mean = loss[valid].sum() / max(1, loss.size)\n    return loss, lse, mean\n\n\ndef pages"),
    # shard statistics: target index not shifted by the shard start
    ("zy[rows] = z[rows, t[rows] - start]", "zy[rows] = z[rows, np.minimum(t[rows], vs - 1)]"),
    # shard statistics: max of the wrong axis
    ("    m = z.max(axis=1)\n    s = np.exp", "    m = z.max(axis=1) * 0.0 + z.max()\n    s = np.exp"),
    # dense CE: drop the stabiliser inside the log but keep it outside
    ("lse = M + np.log(np.exp(z - M[:, None]).sum(axis=1))\n    rows",
     "lse = M + np.log(np.exp(z).sum(axis=1))\n    rows"),
    # gradient: subtract onehot at the wrong column
    ("p[rows, t[rows]] -= 1.0", "p[rows, (t[rows] + 1) % z.shape[1]] -= 1.0"),
    # gradient: forget the ignored rows
    ("    p[~valid] = 0.0\n    return p * g", "    return p * g"),
    # gradient: mean factor over all tokens
    ("return 1.0 / max(1, int((t != ignore_index).sum()))", "return 1.0 / max(1, t.size)"),
    # LM-head backward: transposed operand for dW
    ("return np.matmul(dz, w), np.matmul(dz.T, x)", "return np.matmul(dz, w), np.matmul(x.T, dz).T[::-1]"),
    # LM-head backward: dX from X instead of W
    ("return np.matmul(dz, w), np.matmul(dz.T, x)", "return np.matmul(dz, w) * 2.0, np.matmul(dz.T, x)"),
    # embedding: forget to shift ids to local rows
    ("out[own] = w_shard[ids[own] - start]", "out[own] = w_shard[np.minimum(ids[own], w_shard.shape[0] - 1)]"),
    # embedding: off-by-one at the shard end
    ("own = (ids >= start) & (ids < end)\n    out[own]", "own = (ids >= start) & (ids <= end - 2)\n    out[own]"),
    # shard bounds: accept a non-divisible vocabulary
    ("if V % T != 0:", "if False:"),
    # pages-order CE: no global maximum (per-shard maximum reused)
    ("        S += np.exp(z - m[:, None]).sum(axis=1)", "        S += np.exp(z - z.max(axis=1)[:, None]).sum(axis=1)"),
    # sliced dlogits: missing onehot
    ("    p[rows, t[rows] - start] -= 1.0", "    pass"),
    # two-pass order: sum about the shard's own maximum instead of the given one
    ("    return np.exp(z - np.asarray(m_ref, dtype=np.float64)[:, None]).sum(axis=1)",
     "    return np.exp(z - z.max(axis=1)[:, None]).sum(axis=1)"),
    # padding: round up to a multiple of the per-shard quantum only (not x T)
    ("    q = multiple * T\n", "    q = multiple\n"),
    # padding: round to nearest instead of up
    ("    return -(-V // q) * q", "    return max(q, round(V / q) * q)"),
    # lookup gradient: repeated ids overwrite instead of accumulating
    ("np.add.at(out, ids[own] - start, g[own])", "out[ids[own] - start] = g[own]"),
    # lookup gradient: ids not shifted to local rows
    ("np.add.at(out, ids[own] - start, g[own])", "np.add.at(out, np.minimum(ids[own], end - start - 1), g[own])"),
    # lookup gradient: the shard's first id dropped
    ("own = (ids >= start) & (ids < end)\n    np.add.at", "own = (ids > start) & (ids < end)\n    np.add.at"),
    # chunked shard gradients: each chunk overwrites dW instead of adding to it
    ("        dw += np.matmul(dz.T, x[a:a + chunk])", "        dw = np.matmul(dz.T, x[a:a + chunk])"),
    # chunked shard gradients: dX rows of a chunk stored from the wrong operand
    ("        dx[a:a + chunk] = np.matmul(dz, w)", "        dx[a:a + chunk] = np.matmul(dz, w[::-1])"),
    # lookup gradient rows: id compared without the shard start
    ("sel = np.nonzero(ids == start + int(r))[0]", "sel = np.nonzero(ids == int(r))[0]"),
]


def _mutant(old, new):
    src = inspect.getsource(vp_oracle)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("vp_oracle_mutant")
    exec(compile(src, "vp_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new", MUTATIONS, ids=[f"m{i}" for i in range(len(MUTATIONS))])
def test_mutation_is_caught(old, new):
    mod = _mutant(old, new)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 -- any failure counts as caught
            failed.append(pin.__name__)
    assert failed, "no pin caught the planted mistake"
