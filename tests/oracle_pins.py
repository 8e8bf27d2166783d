"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each ``pin_*`` takes the oracle module as its argument, so the same checks run
on the real oracle (``test_oracle.py``) and on copies of it with a planted
mistake (``test_oracle_mutations.py``, where at least one pin must fail).

What pins what:
  * the pages' worked lookup examples (golden JSON, cited inside each file),
    also run backwards through the lookup's weight gradient;
  * the lookup gradient as the exact adjoint of the lookup (inner products);
  * closed forms of the cross entropy (uniform logits -> log V; a hand-solved
    4-way example) and of its gradient;
  * the identity "sharded statistics merged == dense cross entropy";
  * PyTorch's fp64 ``cross_entropy`` and autograd as an independent textbook
    routine (T = 1, with ignore_index and the mean);
  * central finite differences of the fp64 mean loss;
  * invariants: dlogits rows sum to 0; dX partials sum to the dense dX;
  * a pure-Python loop implementation on tiny inputs.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_problem(seed, N, H, V, scale=1.0, ignore_frac=0.0, ignore_index=-100):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, H))
    w = rng.standard_normal((V, H)) * (scale / np.sqrt(H))
    y = rng.integers(0, V, N).astype(np.int64)
    if ignore_frac:
        y[rng.random(N) < ignore_frac] = ignore_index
    return x, w, y


# ---------------------------------------------------------------------------
def pin_shard_range(o):
    assert o.shard_range(8, 2, 0) == (0, 4) and o.shard_range(8, 2, 1) == (4, 8)
    assert o.shard_range(128256, 8, 0) == (0, 16032)
    assert o.shard_range(152064, 8, 7) == (7 * 19008, 8 * 19008)
    for bad in [(10, 4, 0), (8, 0, 0), (8, 2, 2)]:
        try:
            o.shard_range(*bad)
        except ValueError:
            continue
        raise AssertionError(f"shard_range{bad} must fail")


def pin_padded_vocab(o):
    """The pages' example (50257 -> 51200 for 8 ranks, each shard 6400 = 50 x 128 rows),
    plus the defining properties: divisible, shard rows a multiple of 128, minimal."""
    g = _golden("vocab_padding.json")
    assert o.padded_vocab(g["V"], g["T"], g["multiple"]) == g["V_pad"]
    rng = np.random.default_rng(21)
    for V, T, m in [(8, 2, 1), (16032 * 8, 8, 128), (1, 1, 128), (1000, 3, 128)] + \
            [(int(rng.integers(1, 10**6)), int(rng.integers(1, 17)), int(rng.choice([1, 64, 128, 256])))
             for _ in range(200)]:
        vp = o.padded_vocab(V, T, m)
        assert vp >= V and vp % T == 0 and (vp // T) % m == 0, (V, T, m, vp)
        assert vp - V < m * T, (V, T, m, vp)
        if V % (m * T) == 0:
            assert vp == V
    for bad in [(0, 8, 128), (100, 0, 128), (100, 8, 0)]:
        try:
            o.padded_vocab(*bad)
        except ValueError:
            continue
        raise AssertionError(f"padded_vocab{bad} must fail")


def _check_lookup_golden(o, g):
    V, T, ids = g["V"], g["T"], g["ids"]
    H = 5
    E = (np.arange(V * H, dtype=np.int64).reshape(V, H) + 1)   # distinct non-zero rows
    total = np.zeros((len(ids), H), dtype=np.int64)
    for t in range(T):
        lo, hi = o.shard_range(V, T, t)
        assert [lo, hi] == g["shard_ranges"][t]
        out = o.embed_shard(ids, E[lo:hi], lo, hi)
        for i, src in enumerate(g["per_shard_rows"][str(t)]):
            want = np.zeros(H, dtype=np.int64) if src is None else E[src]
            assert np.array_equal(out[i], want), (t, i)
        total += out
    assert np.array_equal(total, E[g["sum_rows"]])


def pin_embed_worked_example(o):
    _check_lookup_golden(o, _golden("embed_v8_t2_ids_1_6.json"))


def pin_embed_figure1(o):
    _check_lookup_golden(o, _golden("embed_fig1_id5.json"))


def pin_embed_brute(o):
    from oracle import brute
    rng = np.random.default_rng(3)
    V, T, H = 40, 4, 6
    W = rng.integers(0, 65535, (V, H)).astype(np.uint16)
    ids = np.concatenate([rng.integers(-5, V + 5, 50), [-1, 0, 9, 10, 19, 20, 39, 40]])
    dense = np.zeros((ids.size, H), dtype=np.int64)
    for t in range(T):
        lo, hi = o.shard_range(V, T, t)
        got = o.embed_shard(ids, W[lo:hi], lo, hi)
        assert got.dtype == np.uint16
        want = np.array(brute.embed_lookup(ids.tolist(), W[lo:hi].tolist(), lo, hi))
        assert np.array_equal(got.astype(np.int64), want)
        dense += got.astype(np.int64)
    inr = (ids >= 0) & (ids < V)
    assert np.array_equal(dense[inr], W[ids[inr]].astype(np.int64))
    assert not dense[~inr].any()


def pin_embed_grad_brute(o):
    """Weight gradient of the lookup against the pure-Python loops (random ids with
    repeats, off-shard and out-of-range ids)."""
    from oracle import brute
    rng = np.random.default_rng(11)
    V, T, H = 24, 3, 5
    ids = np.concatenate([rng.integers(-3, V + 3, 60), [0, 7, 8, 15, 16, 23, 8, 8]])
    g = rng.standard_normal((ids.size, H))
    for t in range(T):
        lo, hi = o.shard_range(V, T, t)
        got = o.embed_shard_grad(ids, g, lo, hi)
        want = np.array(brute.embed_grad(ids.tolist(), g.tolist(), lo, hi))
        assert got.shape == (hi - lo, H)
        assert np.allclose(got, want, rtol=0, atol=1e-12)


def pin_embed_grad_adjoint(o):
    """The gradient is the adjoint of the (separately pinned) lookup:
    <lookup(ids, W_r), G> == <W_r, grad(ids, G)> on every shard, in fp64."""
    rng = np.random.default_rng(12)
    V, T, H, n = 64, 4, 7, 300
    W = rng.standard_normal((V, H))
    ids = rng.integers(-5, V + 5, n)
    G = rng.standard_normal((n, H))
    for t in range(T):
        lo, hi = o.shard_range(V, T, t)
        lhs = float((o.embed_shard(ids, W[lo:hi], lo, hi) * G).sum())
        rhs = float((W[lo:hi] * o.embed_shard_grad(ids, G, lo, hi)).sum())
        assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs)), (t, lhs, rhs)


def pin_embed_grad_worked_example(o):
    """The V=8, T=2, ids [1, 6] lookup of the pages, run backwards: token 0's gradient
    lands on shard 0's local row 1 and token 1's on shard 1's local row 6 - 4 = 2; the
    shards' gradients side by side are the dense table's gradient (rows 1 and 6)."""
    gfx = _golden("embed_v8_t2_ids_1_6.json")
    V, T, ids = gfx["V"], gfx["T"], gfx["ids"]
    G = np.array([[1.5, -2.0, 0.25], [3.0, 0.5, -1.0]])
    dense = np.zeros((V, 3))
    for t in range(T):
        lo, hi = o.shard_range(V, T, t)
        got = o.embed_shard_grad(ids, G, lo, hi)
        want = np.zeros((hi - lo, 3))
        for i, src in enumerate(gfx["per_shard_rows"][str(t)]):
            if src is not None:
                want[src - lo] += G[i]
        assert np.array_equal(got, want), t
        dense[lo:hi] = got
    assert np.array_equal(dense[1], G[0]) and np.array_equal(dense[6], G[1])
    assert not np.delete(dense, [1, 6], axis=0).any()


def pin_embed_grad_duplicates(o):
    """Repeated ids accumulate; ids outside [0, V) add nothing anywhere."""
    ids = [2, 5, 2, -1, 2, 9, 5, 8, 0]
    G = np.arange(len(ids) * 2, dtype=np.float64).reshape(-1, 2) + 1.0
    lo, hi = 0, 5
    got = o.embed_shard_grad(ids, G, lo, hi)
    want = np.zeros((5, 2))
    want[2] = G[0] + G[2] + G[4]
    want[0] = G[8]
    assert np.array_equal(got, want)
    got1 = o.embed_shard_grad(ids, G, 5, 10)
    want1 = np.zeros((5, 2))
    want1[0] = G[1] + G[6]
    want1[4] = G[5]
    want1[3] = G[7]
    assert np.array_equal(got1, want1)
    rows = [2, 4, 0]
    assert np.array_equal(o.embed_shard_grad_rows(ids, G, 5, rows), got1[rows])
    assert np.array_equal(o.embed_shard_grad_rows(ids, G, 0, rows), got[rows])


def pin_uniform_logits(o):
    g = _golden("ce_closed_forms.json")["uniform"]
    for case in g["cases"][:1]:
        V = case["V"]
        N, H = 7, 4
        x = np.random.default_rng(0).standard_normal((N, H))
        w = np.zeros((V, H))
        y = np.arange(N) % V
        for T in (1, 2, 4, 8, 16):
            if V % T:
                continue
            m, s, zy = [], [], []
            for t in range(T):
                lo, hi = o.shard_range(V, T, t)
                a, b, c = o.shard_stats(o.logits(x, w[lo:hi]), y, lo)
                m.append(a), s.append(b), zy.append(c)
            loss, lse, mean = o.combine_triples(np.array(m), np.array(s), np.array(zy), y)
            assert np.allclose(loss, case["loss"], rtol=0, atol=1e-12)
            assert abs(mean - case["loss"]) < 1e-12
        loss, lse, mean = o.dense_ce(o.logits(x, w), y)
        assert np.allclose(loss, case["loss"], rtol=0, atol=1e-12)
        dz = o.dense_dlogits(o.logits(x, w), y)
        want = np.full((N, V), 1.0 / V)
        want[np.arange(N), y] -= 1.0
        assert np.allclose(dz, want / N, rtol=0, atol=1e-15)


def pin_geometric(o):
    g = _golden("ce_closed_forms.json")["geometric"]
    z = np.array([g["logits"]])
    y = np.array([g["target"]])
    loss, lse, mean = o.dense_ce(z, y)
    assert abs(loss[0] - g["loss"]) < 1e-13 and abs(mean - g["loss"]) < 1e-13
    assert abs(lse[0] - np.log(10.0)) < 1e-13
    assert np.allclose(o.dense_dlogits(z, y)[0], g["dlogits"], rtol=0, atol=1e-14)
    # the same example split over two shards of two columns each
    m, s, zy = zip(*[o.shard_stats(z[:, lo:lo + 2], y, lo) for lo in (0, 2)])
    l2, lse2, _ = o.combine_triples(np.array(m), np.array(s), np.array(zy), y)
    assert abs(l2[0] - g["loss"]) < 1e-13 and abs(lse2[0] - np.log(10.0)) < 1e-13
    l3, _, _ = o.pages_sharded_ce([z[:, :2], z[:, 2:]], y, [0, 2])
    assert abs(l3[0] - g["loss"]) < 1e-13


def pin_sharded_equals_dense(o):
    """The pages' NumPy check (n=6, V=16, t=4, logits ~ N(0,1)*5) plus wider splits."""
    for seed, (N, V) in enumerate([(6, 16), (33, 48), (20, 64)]):
        rng = np.random.default_rng(seed)
        z = rng.standard_normal((N, V)) * 5
        y = rng.integers(0, V, N)
        y[::7] = -100
        ref, ref_lse, ref_mean = o.dense_ce(z, y)
        for T in (1, 2, 4, 8, 16):
            if V % T:
                continue
            Vs = V // T
            shards = [z[:, t * Vs:(t + 1) * Vs] for t in range(T)]
            starts = [t * Vs for t in range(T)]
            m, s, zy = zip(*[o.shard_stats(zz, y, lo) for zz, lo in zip(shards, starts)])
            loss, lse, mean = o.combine_triples(np.array(m), np.array(s), np.array(zy), y)
            assert np.allclose(loss, ref, rtol=0, atol=1e-12)
            assert np.allclose(lse, ref_lse, rtol=0, atol=1e-12)
            assert abs(mean - ref_mean) < 1e-12
            l2, lse2, mean2 = o.pages_sharded_ce(shards, y, starts)
            assert np.allclose(l2, ref, rtol=0, atol=1e-12)
            assert abs(mean2 - ref_mean) < 1e-12


def pin_shard_sumexp_two_pass(o):
    """The pages' two-pass order from per-shard pieces: the global max of the shards' local
    maxima, then each shard's sum about it; their total reproduces the dense lse, and merged
    with the combine (every shard's max set to the global one) the dense loss."""
    x, w, y = _rand_problem(31, 40, 12, 60, scale=4.0, ignore_frac=0.1)
    z = o.logits(x, w)
    loss, lse, mean = o.dense_ce(z, y)
    T = 5
    bounds = [o.shard_range(60, T, t) for t in range(T)]
    M = np.max(np.stack([o.shard_stats(z[:, a:b], y, a)[0] for a, b in bounds]), axis=0)
    assert np.allclose(M, z.max(axis=1), rtol=0, atol=0)
    s = np.stack([o.shard_sumexp(z[:, a:b], M) for a, b in bounds])
    assert np.allclose(M + np.log(s.sum(axis=0)), lse, rtol=0, atol=1e-12)
    zy = np.stack([o.shard_stats(z[:, a:b], y, a)[2] for a, b in bounds])
    l2, lse2, mean2 = o.combine_triples(np.broadcast_to(M, s.shape), s, zy, y)
    assert np.allclose(l2, loss, rtol=0, atol=1e-12) and abs(mean2 - mean) < 1e-12


def pin_torch_cross_entropy(o):
    import torch
    import torch.nn.functional as F
    x, w, y = _rand_problem(11, 37, 24, 50, scale=4.0, ignore_frac=0.2)
    loss, lse, mean = o.dense_ce(o.logits(x, w), y)
    zt = torch.from_numpy(x) @ torch.from_numpy(w).T
    tl = F.cross_entropy(zt, torch.from_numpy(y), ignore_index=-100, reduction="none")
    tm = F.cross_entropy(zt, torch.from_numpy(y), ignore_index=-100, reduction="mean")
    assert np.allclose(loss, tl.numpy(), rtol=0, atol=1e-12)
    assert abs(mean - tm.item()) < 1e-12
    assert np.allclose(lse, torch.logsumexp(zt, 1).numpy(), rtol=0, atol=1e-12)


def pin_torch_autograd(o):
    import torch
    import torch.nn.functional as F
    x, w, y = _rand_problem(12, 29, 16, 40, scale=3.0, ignore_frac=0.25)
    xt = torch.from_numpy(x).requires_grad_(True)
    wt = torch.from_numpy(w).requires_grad_(True)
    F.cross_entropy(xt @ wt.T, torch.from_numpy(y), ignore_index=-100).backward()
    dz = o.dense_dlogits(o.logits(x, w), y)
    dx, dw = o.shard_grads(x, w, dz)
    assert np.allclose(dx, xt.grad.numpy(), rtol=0, atol=1e-13)
    assert np.allclose(dw, wt.grad.numpy(), rtol=0, atol=1e-13)


def pin_finite_differences(o):
    x, w, y = _rand_problem(13, 6, 8, 16, scale=5.0, ignore_frac=0.0)
    y[1] = -100

    def L(xx, ww):
        return o.dense_ce(o.logits(xx, ww), y)[2]

    dz = o.dense_dlogits(o.logits(x, w), y)
    dx, dw = o.shard_grads(x, w, dz)
    h = 1e-6
    rng = np.random.default_rng(0)
    for _ in range(12):
        i, k = rng.integers(0, x.shape[0]), rng.integers(0, x.shape[1])
        xp, xm = x.copy(), x.copy()
        xp[i, k] += h
        xm[i, k] -= h
        assert abs((L(xp, w) - L(xm, w)) / (2 * h) - dx[i, k]) < 1e-7
        j, k = rng.integers(0, w.shape[0]), rng.integers(0, w.shape[1])
        wp, wm = w.copy(), w.copy()
        wp[j, k] += h
        wm[j, k] -= h
        assert abs((L(x, wp) - L(x, wm)) / (2 * h) - dw[j, k]) < 1e-7


def pin_dlogits_invariants(o):
    x, w, y = _rand_problem(14, 40, 12, 64, scale=6.0, ignore_frac=0.2)
    dz = o.dense_dlogits(o.logits(x, w), y)
    valid = y != -100
    assert np.allclose(dz.sum(axis=1), 0.0, atol=1e-15)
    assert not dz[~valid].any()
    # the only negative entry of a valid row sits at the target
    neg = dz < 0
    assert np.array_equal(np.nonzero(neg)[1], y[np.nonzero(neg)[0]])
    # all ignored: mean 0 and zero gradient (max(1, N_valid) guard)
    yi = np.full_like(y, -100)
    loss, _, mean = o.dense_ce(o.logits(x, w), yi)
    assert mean == 0.0 and not loss.any()
    assert not o.dense_dlogits(o.logits(x, w), yi).any()


def pin_dx_partials_sum(o):
    x, w, y = _rand_problem(15, 25, 10, 48, scale=4.0, ignore_frac=0.1)
    dz = o.dense_dlogits(o.logits(x, w), y)
    dx, dw = o.shard_grads(x, w, dz)
    for T in (2, 4, 8):
        Vs = 48 // T
        parts = [o.shard_grads(x, w[t * Vs:(t + 1) * Vs], dz[:, t * Vs:(t + 1) * Vs])
                 for t in range(T)]
        assert np.allclose(sum(p[0] for p in parts), dx, rtol=0, atol=1e-13)
        assert np.allclose(np.concatenate([p[1] for p in parts]), dw, rtol=0, atol=1e-14)


def pin_brute_loops(o):
    from oracle import brute
    x, w, y = _rand_problem(16, 6, 8, 16, scale=5.0)
    y[4] = -100
    z, loss, mean, dz, dx, dw = brute.ce_loss_and_grads(x.tolist(), w.tolist(), y.tolist())
    zo = o.logits(x, w)
    assert np.allclose(zo, z, rtol=0, atol=1e-12)
    lo, _, mo = o.dense_ce(zo, y)
    assert np.allclose(lo, loss, rtol=0, atol=1e-12) and abs(mo - mean) < 1e-12
    dzo = o.dense_dlogits(zo, y)
    assert np.allclose(dzo, dz, rtol=0, atol=1e-14)
    dxo, dwo = o.shard_grads(x, w, dzo)
    assert np.allclose(dxo, dx, rtol=0, atol=1e-13) and np.allclose(dwo, dw, rtol=0, atol=1e-13)


def pin_sliced_helpers(o):
    x, w, y = _rand_problem(17, 70, 16, 96, scale=5.0, ignore_frac=0.1)
    z = o.logits(x, w)
    loss, lse, mean = o.dense_ce(z, y)
    assert np.allclose(o.lse_dense_chunked(x, w, chunk=16), lse, rtol=0, atol=1e-12)
    g = o.mean_scale(y)
    dz = o.dense_dlogits(z, y)
    lo, hi = 32, 64
    a = o.shard_stats(z[:, lo:hi], y, lo)
    b = o.shard_stats_chunked(x, w[lo:hi], y, lo, chunk=9)
    for u, v in zip(a, b):
        assert np.allclose(u, v, rtol=0, atol=1e-12)
    rows = np.array([0, 5, 69, 33])
    assert np.allclose(o.dz_rows(x[rows], w[lo:hi], y[rows], lse[rows], lo, g), dz[rows, lo:hi],
                       rtol=0, atol=1e-15)
    cols = np.array([0, 40, 95, 63])
    assert np.allclose(o.dz_cols(x, w[cols], cols, y, lse, g), dz[:, cols], rtol=0, atol=1e-15)
    # whole-shard gradients from token chunks (a ragged last chunk) == the dense ones
    dxr, dwr = o.shard_grads(x, w[lo:hi], dz[:, lo:hi])
    dxc, dwc = o.shard_grads_chunked(x, w[lo:hi], y, lse, lo, g, chunk=16)
    assert np.allclose(dxc, dxr, rtol=0, atol=1e-14) and np.allclose(dwc, dwr, rtol=0, atol=1e-14)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
