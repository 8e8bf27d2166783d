"""Pure-Python loop version of the cross entropy and its gradients, for tiny inputs.

TEST INFRASTRUCTURE (same rules as ``vp_oracle``).  Written with plain loops
and the ``math`` module only -- no NumPy -- so that it shares no routine with
``vp_oracle`` and can cross-check it element by element on inputs of a few
hundred values.

Definitions ("5 Vocab Parallelism", 5.3.1-5.3.3; interview note "Vocab
parallelism", key formulas and backward):
  z[n][j]  = sum_k x[n][k] * w[j][k]
  loss_n   = log(sum_j exp(z[n][j])) - z[n][y_n]      (0 if y_n is ignored)
  L        = sum_valid loss_n / max(1, N_valid)
  dz[n][j] = (softmax(z_n)_j - [j == y_n]) / max(1, N_valid)   (0 if ignored)
  dX       = dz W,  dW = dz^T X
"""
from __future__ import annotations

import math


def ce_loss_and_grads(x, w, targets, ignore_index=-100):
    """x: N lists of H floats, w: V lists of H floats, targets: N ints."""
    N, V, H = len(x), len(w), len(w[0])
    z = [[sum(x[n][k] * w[j][k] for k in range(H)) for j in range(V)] for n in range(N)]
    nvalid = sum(1 for y in targets if y != ignore_index)
    scale = 1.0 / max(1, nvalid)
    loss = [0.0] * N
    dz = [[0.0] * V for _ in range(N)]
    for n in range(N):
        y = targets[n]
        if y == ignore_index:
            continue
        mx = max(z[n])
        tot = sum(math.exp(v - mx) for v in z[n])
        loss[n] = math.log(tot) + mx - z[n][y]
        for j in range(V):
            p = math.exp(z[n][j] - mx) / tot
            dz[n][j] = (p - (1.0 if j == y else 0.0)) * scale
    mean = sum(loss) / max(1, nvalid)
    dx = [[sum(dz[n][j] * w[j][k] for j in range(V)) for k in range(H)] for n in range(N)]
    dw = [[sum(dz[n][j] * x[n][k] for n in range(N)) for k in range(H)] for j in range(V)]
    return z, loss, mean, dz, dx, dw


def embed_lookup(ids, w_rows, start, end):
    """Per-shard lookup: the local row for owned ids, a zero row otherwise (5.2.1)."""
    H = len(w_rows[0])
    out = []
    for i in ids:
        if start <= i < end:
            out.append(list(w_rows[i - start]))
        else:
            out.append([0] * H)
    return out


def embed_grad(ids, dout_rows, start, end):
    """Weight gradient of the per-shard lookup: each owned token adds its gradient row
    to local row id - start (the adjoint of ``embed_lookup``)."""
    H = len(dout_rows[0])
    out = [[0.0] * H for _ in range(end - start)]
    for i, tok_id in enumerate(ids):
        if start <= tok_id < end:
            row = out[tok_id - start]
            for k in range(H):
                row[k] += dout_rows[i][k]
    return out
