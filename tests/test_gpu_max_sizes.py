"""The largest sizes the C ABI accepts, one dimension at a time, against the oracle.

The CE path takes N, H and Vs up to 2^20 each.  At those sizes a GEMM operand row
is 2 MiB of bf16 and a 256-row fp32 output panel just under 1 GiB, which is where
the kernels' buffer resources (capped at 1 GiB) and 32-bit offsets come closest to
their limits; a K loop of 16384 steps, a vocabulary of 8192 statistics slices and
grids of 4096 tiles along one side are exercised too.  The lookup gradient takes up
to 2^24 ids (a radix sort over 16384 tiles).  Same bars as the other parity tests.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import vp_inputs
from gpu_util import (assert_grad_close, assert_loss_close, assert_stats_close, dev_bf16, dev_i64,
                      embed_bwd_compare, embed_bwd_run, host, log, run_ce_path)

pytestmark = pytest.mark.gpu

MAX = 1 << 20


@pytest.fixture(scope="module")
def vp():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_lm_head_amd
    return vocab_lm_head_amd


def _bf16_normal(r, shape, scale):
    """bf16 bits of N(0, scale^2) values, drawn from a table of 65536 such values (the
    sizes here make a full fp32 draw and rounding take minutes on the host)."""
    table = vp_inputs.f32_to_bf16_bits(r.standard_normal(1 << 16, dtype=np.float32) * np.float32(scale))
    return table[r.integers(0, 1 << 16, size=shape, dtype=np.uint16, endpoint=False)]


def _check(vp, xb, wb, y, T, bwd_shards, label):
    """Every shard's forward, the combine and the given shards' backward, all on the
    GPU, against the dense oracle: statistics, loss, lse and mean of every token, dX
    partials and dW in full."""
    import torch
    N, H = xb.shape
    V = wb.shape[0]
    log(f"  case {label}: N={N} H={H} V={V} T={T}")
    x, w = vp_inputs.bf16_bits_to_f64(xb), vp_inputs.bf16_bits_to_f64(wb)
    z = oracle.logits(x, w)
    loss, lse, mean = oracle.dense_ce(z, y)
    g = oracle.mean_scale(y)
    rng = [oracle.shard_range(V, T, t) for t in range(T)]
    x_d, w_d, y_d = dev_bf16(xb), dev_bf16(wb), dev_i64(y)
    out = run_ce_path(vp, x_d, [w_d[a:b] for a, b in rng], [a for a, _ in rng],
                      [b for _, b in rng], y_d, g, bwd_shards=bwd_shards)
    for t, (a, b) in enumerate(rng):
        assert_stats_close((host(out["m"][t]), host(out["s"][t]), host(out["zy"][t])),
                           oracle.shard_stats(z[:, a:b], y, a), f"shard {t} stats")
    assert_loss_close(host(out["loss"]), loss)
    assert_loss_close(host(out["lse"]), lse, "lse")
    assert abs(float(out["mean"].item()) - mean) <= 2e-3
    dz = oracle.dense_dlogits(z, y)
    del z
    for t in bwd_shards:
        a, b = rng[t]
        dxr, dwr = oracle.shard_grads(x, w[a:b], dz[:, a:b])
        assert_grad_close(host(out["grads"][t][0]), dxr, f"dX partial {t}")
        assert_grad_close(host(out["grads"][t][1]), dwr, f"dW {t}")
        out["grads"][t] = None
        torch.cuda.empty_cache()


def test_max_vocab_rows(vp):
    """One shard of 2^20 vocabulary rows (V = 2^20, T = 1), 64 tokens, H = 64; targets on
    both ends of the shard and 10% ignored."""
    r = np.random.default_rng(20)
    N, H, V = 64, 64, MAX
    xb = _bf16_normal(r, (N, H), 1.0)
    wb = _bf16_normal(r, (V, H), 3.0 / math.sqrt(H))
    y = r.integers(0, V, N).astype(np.int64)
    y[:2] = [0, V - 1]
    y[r.random(N) < 0.1] = -100
    _check(vp, xb, wb, y, T=1, bwd_shards=[0], label="Vs = 2^20")


def test_max_tokens(vp):
    """2^20 tokens, V = 64 in two shards of 32, H = 64; shard 1's backward."""
    r = np.random.default_rng(21)
    N, H, V = MAX, 64, 64
    xb = _bf16_normal(r, (N, H), 1.0)
    wb = _bf16_normal(r, (V, H), 3.0 / math.sqrt(H))
    y = r.integers(0, V, N).astype(np.int64)
    y[r.random(N) < 0.05] = -100
    _check(vp, xb, wb, y, T=2, bwd_shards=[1], label="N = 2^20")


def test_max_hidden(vp):
    """H = 2^20: K loops of 16384 steps and, with 256 tokens, a dX panel of 256 rows x
    2^20 fp32 columns (1 GiB: its last stores come closest to the buffer resource's
    end).  V = 16 in two shards, both backwards.  X is zero outside 384 columns (the
    first, middle and last 128), so that the oracle needs only those columns of X -- a
    zero column adds exact zeros to every product it enters -- while the kernels still
    stream all of it; W is dense.  dX is compared on 18 token rows (the first and last
    among them) across all 2^20 columns, dW in full."""
    import torch
    r = np.random.default_rng(22)
    N, H, V, T = 256, MAX, 16, 2
    cols = np.concatenate([np.arange(128), np.arange(H // 2 - 64, H // 2 + 64),
                           np.arange(H - 128, H)])
    xb = np.zeros((N, H), dtype=np.uint16)
    xb[:, cols] = _bf16_normal(r, (N, cols.size), 1.0)
    wb = _bf16_normal(r, (V, H), 3.0 / math.sqrt(cols.size))
    y = r.integers(0, V, N).astype(np.int64)
    log(f"  case H = 2^20: N={N} V={V} T={T}, X nonzero in {cols.size} columns")
    xs = vp_inputs.bf16_bits_to_f64(xb[:, cols])
    w = vp_inputs.bf16_bits_to_f64(wb)
    z = oracle.logits(xs, w[:, cols])
    loss, lse, mean = oracle.dense_ce(z, y)
    g = oracle.mean_scale(y)
    rng = [oracle.shard_range(V, T, t) for t in range(T)]
    x_d, w_d, y_d = dev_bf16(xb), dev_bf16(wb), dev_i64(y)
    out = run_ce_path(vp, x_d, [w_d[a:b] for a, b in rng], [a for a, _ in rng],
                      [b for _, b in rng], y_d, g, bwd_shards=list(range(T)))
    del x_d
    for t, (a, b) in enumerate(rng):
        assert_stats_close((host(out["m"][t]), host(out["s"][t]), host(out["zy"][t])),
                           oracle.shard_stats(z[:, a:b], y, a), f"shard {t} stats")
    assert_loss_close(host(out["loss"]), loss)
    assert_loss_close(host(out["lse"]), lse, "lse")
    assert abs(float(out["mean"].item()) - mean) <= 2e-3
    dz = oracle.dense_dlogits(z, y)
    rows = np.unique(np.concatenate([r.choice(N, 16, replace=False), [0, N - 1]]))
    for t, (a, b) in enumerate(rng):
        dxr = oracle.shard_grads(xs[rows], w[a:b], dz[rows, a:b])[0]
        got_dx = host(out["grads"][t][0][torch.from_numpy(rows).cuda()])
        assert_grad_close(got_dx, dxr, f"dX partial {t} ({rows.size} rows)")
        dwr = np.zeros((b - a, H))
        dwr[:, cols] = oracle.shard_grads(xs, w[a:b][:, cols], dz[:, a:b])[1]
        assert_grad_close(host(out["grads"][t][1]), dwr, f"dW {t}")
        out["grads"][t] = None
        torch.cuda.empty_cache()


def test_max_lookup_gradient_ids(vp):
    """2^24 ids, the lookup gradient's limit (a radix sort over 16384 tiles): uniform ids
    over V = 1600000 (and a few outside it) plus one row named 2^21 times, on shard 1
    of 16 ([100000, 8]), added into a random prefill; every row of the shard against
    the oracle.  Only owned tokens' gradient rows are read, so only those are drawn
    (the others are zero) and handed to the oracle."""
    r = np.random.default_rng(23)
    n, h, V, T = 1 << 24, 8, 1600000, 16
    lo, hi = vp.vp_shard_range(V, T, 1)
    ids = np.concatenate([r.integers(-5, V + 5, n - (1 << 21)),
                          np.full(1 << 21, lo + 12345)]).astype(np.int64)
    r.shuffle(ids)
    own = (ids >= lo) & (ids < hi)
    dout = np.zeros((n, h), dtype=np.uint16)
    dout[own] = _bf16_normal(r, (int(own.sum()), h), 1.0)
    dw0 = r.standard_normal((hi - lo, h)).astype(np.float32)
    log(f"  case 2^24 ids: n={n} h={h} rows={hi - lo}, {int(own.sum())} owned")
    got = host(embed_bwd_run(vp, ids, dout, lo, hi, dw0))
    d = vp_inputs.bf16_bits_to_f64(dout[own])
    count = np.bincount(ids[own] - lo, minlength=hi - lo).astype(np.float64)
    embed_bwd_compare(got, dw0, oracle.embed_shard_grad(ids[own], d, lo, hi),
                      oracle.embed_shard_grad(ids[own], np.abs(d), lo, hi), count, "2^24 ids")
