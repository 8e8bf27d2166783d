"""A seeded sweep of 24 random small shapes through the whole CE path, each compared in full
with the oracle: odd N, H (a multiple of 8) and Vs, T = 1..5, 10% ignored targets.  The
shapes are drawn so that the forward's slice merge runs in one pass and split 2-5 ways,
and the gradient GEMMs run as 128 x 128 tiles in one launch (18 shapes) or, for the wide
shards, split over K (6), in many combinations.
A second sweep of 24 random shapes covers the lookup and its gradient.
Same bars as the other parity tests."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import vp_inputs
from gpu_util import (assert_grad_close, assert_loss_close, assert_stats_close, dev_bf16, dev_i64,
                      host, log, run_ce_path)

pytestmark = pytest.mark.gpu


def _cases():
    r = np.random.default_rng(2024)
    out = []
    for i in range(24):
        T = int(r.integers(1, 6))
        if i % 4 == 0:     # few tokens, a wide shard: the merge splits, dX splits over K
            N, H, Vs = int(r.integers(1, 200)), 8 * int(r.integers(1, 17)), int(r.integers(8000, 24000))
            T = min(T, 2)
        elif i % 4 == 1:   # many tokens, a narrow shard
            N, H, Vs = int(r.integers(1000, 3000)), 8 * int(r.integers(1, 65)), int(r.integers(1, 1500))
        elif i % 4 == 2:
            N, H, Vs = int(r.integers(1, 700)), 8 * int(r.integers(1, 129)), int(r.integers(1, 3000))
        else:
            N, H, Vs = int(r.integers(300, 1500)), 8 * int(r.integers(8, 65)), int(r.integers(1000, 4000))
        out.append((i, N, H, Vs, T))
    return out


@pytest.fixture(scope="module")
def vp():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_lm_head_amd
    return vocab_lm_head_amd


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"{c[0]}-N{c[1]}-H{c[2]}-Vs{c[3]}-T{c[4]}")
def test_random_shape(vp, case):
    i, N, H, Vs, T = case
    V = Vs * T
    r = np.random.default_rng(1000 + i)
    xb = vp_inputs.f32_to_bf16_bits(r.standard_normal((N, H)).astype(np.float32))
    wb = vp_inputs.f32_to_bf16_bits(
        r.standard_normal((V, H)).astype(np.float32) * np.float32(3.0 / math.sqrt(H)))
    y = r.integers(0, V, N).astype(np.int64)
    y[r.random(N) < 0.1] = oracle.DEFAULT_IGNORE_INDEX
    log(f"  case {i}: N={N} H={H} Vs={Vs} T={T}")
    x, w = vp_inputs.bf16_bits_to_f64(xb), vp_inputs.bf16_bits_to_f64(wb)
    z = oracle.logits(x, w)
    loss, lse, mean = oracle.dense_ce(z, y)
    dz = oracle.dense_dlogits(z, y)
    g = oracle.mean_scale(y)
    rng = [oracle.shard_range(V, T, t) for t in range(T)]
    x_d, w_d, y_d = dev_bf16(xb), dev_bf16(wb), dev_i64(y)
    out = run_ce_path(vp, x_d, [w_d[a:b] for a, b in rng], [a for a, _ in rng],
                      [b for _, b in rng], y_d, g, bwd_shards=range(T))
    for t, (a, b) in enumerate(rng):
        assert_stats_close((host(out["m"][t]), host(out["s"][t]), host(out["zy"][t])),
                           oracle.shard_stats(z[:, a:b], y, a), f"shard {t} stats")
    assert_loss_close(host(out["loss"]), loss)
    assert_loss_close(host(out["lse"]), lse, "lse")
    assert abs(float(out["mean"].item()) - mean) <= 2e-3
    for t, (a, b) in enumerate(rng):
        dxr, dwr = oracle.shard_grads(x, w[a:b], dz[:, a:b])
        assert_grad_close(host(out["grads"][t][0]), dxr, f"dX partial {t}")
        assert_grad_close(host(out["grads"][t][1]), dwr, f"dW {t}")


def _lookup_cases():
    """Seeded shapes for the lookup and its gradient: n 1-12000, h a multiple of 8 up to
    2400 (one to five 512-column blocks, most of them ragged), Vs 1-100000 (one, two or
    three 8-bit radix passes), ids mixed from four sources: uniform over the shard and
    a margin around it, Zipf-like repeats, a few very hot rows that cross many 64-position
    blocks, and negative or ignored ids."""
    r = np.random.default_rng(77)
    out = []
    for i in range(24):
        n = int(np.exp(r.uniform(0.0, np.log(12000))))
        h = 8 * int(r.integers(1, 301))
        vs = int(np.exp(r.uniform(0.0, np.log(100000))))
        if i % 6 == 0:                       # keys past 16 bits: three radix passes
            vs = int(r.integers(65536, 100001))
        if i % 4 == 1:                       # several sort tiles
            n = int(r.integers(4000, 12001))
        if i == 23:                          # a one-row shard
            vs = 1
        if vs * h > 4 << 20:                 # keep the fp64 oracle small
            h = max(8, 8 * ((4 << 20) // (vs * 8)))
        n = min(n, max(1, (8 << 20) // h))
        lo = int(r.integers(0, 1000))
        out.append((i, n, h, lo, lo + vs))
    return out


def _lookup_ids(r, n, lo, hi):
    vs = hi - lo
    margin = vs // 4 + 3
    kind = r.integers(0, 4, n)
    uni = r.integers(lo - margin, hi + margin, n)
    perm = r.permutation(vs)
    zipf = lo + perm[np.minimum(r.zipf(1.1, n), vs) - 1]
    hot = lo + perm[r.integers(0, min(3, vs), n)]
    neg = np.where(r.random(n) < 0.5, -100, -1 - r.integers(0, 1 << 40, n))
    ids = np.choose(kind, [uni, zipf, hot, neg])
    return ids.astype(np.int64)


@pytest.mark.parametrize("case", _lookup_cases(),
                         ids=lambda c: f"{c[0]}-n{c[1]}-h{c[2]}-Vs{c[4] - c[3]}")
def test_random_lookup_shape(vp, case):
    """The lookup bit for bit, and its gradient added into a prefilled (or zero) dw
    within the summation bound on every row, untouched rows unchanged."""
    from gpu_util import bf16_bits, embed_bwd_full_check
    i, n, h, lo, hi = case
    r = np.random.default_rng(3000 + i)
    ids = _lookup_ids(r, n, lo, hi)
    log(f"  case {i}: n={n} h={h} rows={hi - lo} owned={int(((ids >= lo) & (ids < hi)).sum())}")
    wb = vp_inputs.f32_to_bf16_bits(r.standard_normal((hi - lo, h)).astype(np.float32))
    got = bf16_bits(vp.vp_embed_fwd(dev_i64(ids), dev_bf16(wb), lo, hi))
    assert np.array_equal(got, oracle.embed_shard(ids, wb, lo, hi)), "lookup differs"
    dout = vp_inputs.f32_to_bf16_bits(r.standard_normal((n, h)).astype(np.float32))
    dw0 = (r.standard_normal((hi - lo, h)).astype(np.float32) if i % 2
           else np.zeros((hi - lo, h), np.float32))
    embed_bwd_full_check(vp, ids, dout, lo, hi, dw0, f"lookup gradient case {i}")
