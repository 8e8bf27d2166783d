"""The materialised-logits comparator (stored fp32 logits, the pages' order of the
statistics, backward from the stored logits) against the oracle, through the C ABI.
Same bars as the fused path: loss / lse / statistics abs 2e-3 (s relative), dX and dW
max relative 1e-2; stored logits abs 2e-3 (fp32 sums of bf16 products, K <= 4096)."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import vp_inputs
from gpu_util import (assert_grad_close, assert_loss_close, assert_stats_close, dev_bf16, dev_i64,
                      full_grads, host, log)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vp():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_lm_head_amd
    return vocab_lm_head_amd


def _comparator(vp, x_d, w_shards, starts, ends, y_d, g, two_pass, bwd_shards):
    """Every shard's logits and statistics (one read, or the pages' two passes), combine,
    then the selected shards' backward from their stored logits."""
    import torch
    n = x_d.shape[0]
    T = len(w_shards)
    logits = [vp.vp_lmhead_logits(x_d, w_shards[t], starts[t], ends[t]) for t in range(T)]
    m = torch.empty((T, n), dtype=torch.float32, device="cuda")
    s, zy = torch.empty_like(m), torch.empty_like(m)
    for t in range(T):
        vp.vp_logits_ce_stats(logits[t], y_d, starts[t], ends[t], None, m[t], s[t], zy[t])
    if two_pass:   # all-reduce MAX, then every shard's sum about the global maximum
        M = vp.vp_ce_max(m)
        for t in range(T):
            vp.vp_logits_ce_stats(logits[t], y_d, starts[t], ends[t], M, m[t], s[t], zy[t])
    loss, lse, mean = vp.vp_ce_combine(m, s, zy, y_d)
    grads = {t: vp.vp_logits_ce_bwd(logits[t], x_d, w_shards[t], y_d, lse, starts[t], ends[t], g)
             for t in bwd_shards}
    torch.cuda.synchronize()
    return {"logits": logits, "m": m, "s": s, "zy": zy, "loss": loss, "lse": lse, "mean": mean,
            "grads": grads}


def _full_check(vp, xb, wb, y, T, two_pass, label):
    N, H = xb.shape
    V = wb.shape[0]
    x, w = vp_inputs.bf16_bits_to_f64(xb), vp_inputs.bf16_bits_to_f64(wb)
    z = oracle.logits(x, w)
    loss, lse, mean = oracle.dense_ce(z, y)
    dz = oracle.dense_dlogits(z, y)
    g = oracle.mean_scale(y)
    rng = [oracle.shard_range(V, T, t) for t in range(T)]
    x_d, w_d, y_d = dev_bf16(xb), dev_bf16(wb), dev_i64(y)
    log(f"  comparator {label}: N={N} H={H} V={V} T={T} two_pass={two_pass}")
    out = _comparator(vp, x_d, [w_d[a:b] for a, b in rng], [a for a, _ in rng], [b for _, b in rng],
                      y_d, g, two_pass, range(T))
    M = z.max(axis=1)
    for t, (a, b) in enumerate(rng):
        lg = host(out["logits"][t])
        assert lg.shape[1] == vp.logits_ld(b - a)
        err = float(np.abs(lg[:, :b - a] - z[:, a:b]).max())
        assert err <= 2e-3, f"shard {t} logits err {err}"
        assert not lg[:, b - a:].any(), "padding columns of the stored logits must be zero"
        if two_pass:
            want = (M, oracle.shard_sumexp(z[:, a:b], M), oracle.shard_stats(z[:, a:b], y, a)[2])
        else:
            want = oracle.shard_stats(z[:, a:b], y, a)
        assert_stats_close((host(out["m"][t]), host(out["s"][t]), host(out["zy"][t])), want,
                           f"shard {t} stats")
    assert_loss_close(host(out["loss"]), loss)
    assert_loss_close(host(out["lse"]), lse, "lse")
    assert abs(float(out["mean"].item()) - mean) <= 2e-3
    for t, (a, b) in enumerate(rng):
        dxr, dwr = oracle.shard_grads(x, w[a:b], dz[:, a:b])
        assert_grad_close(host(out["grads"][t][0]), dxr, f"dX partial {t}")
        assert_grad_close(host(out["grads"][t][1]), dwr, f"dW {t}")


@pytest.mark.parametrize("two_pass", [False, True])
def test_small_lm(vp, two_pass):
    """N=4096, H=512, V=6400, T=2: every stored logit, both orders of the statistics,
    loss and both shards' gradients."""
    inp = vp_inputs.make_inputs("small_lm")
    _full_check(vp, inp.x, inp.w, inp.targets, inp.wl.T, two_pass, "small_lm")


def test_ragged_shards_and_rows(vp):
    """Vs = 334 (not a multiple of 4: stored rows padded to 336), N = 300, H = 64, T = 3,
    targets on every shard's first and last row and 10% ignored."""
    r = np.random.default_rng(334)
    N, H, V, T = 300, 64, 1002, 3
    xb = vp_inputs.f32_to_bf16_bits(r.standard_normal((N, H)).astype(np.float32))
    wb = vp_inputs.f32_to_bf16_bits(
        r.standard_normal((V, H)).astype(np.float32) * (4.0 / math.sqrt(H)))
    y = r.integers(0, V, N).astype(np.int64)
    y[:6] = [0, 333, 334, 667, 668, 1001]
    y[r.random(N) < 0.1] = -100
    _full_check(vp, xb, wb, y, T, True, "ragged")


@pytest.mark.timeout(900)
def test_shard_8b_against_golden(vp):
    """The 8B-class shard 0 ([16032, 4096], N = 8192), statistics in one read: every token's
    loss and lse against the oracle golden (shards 1..7's statistics from their fused
    forwards, other GPUs' work), 24 stored-logit rows, and sampled dX and dW rows against
    the oracle."""
    import os

    import torch
    inp = vp_inputs.make_inputs("shard_8b", shards=[0])
    wl = inp.wl
    y = inp.targets
    gold = np.load(os.path.join(os.path.dirname(__file__), "golden", "oracle_shard_8b.npz"))
    x_d, y_d = dev_bf16(inp.x), dev_i64(y)
    lo, hi = vp.vp_shard_range(wl.V, wl.T, 0)
    w0 = dev_bf16(inp.w[lo:hi])
    m = torch.empty((wl.T, wl.N), dtype=torch.float32, device="cuda")
    s, zy = torch.empty_like(m), torch.empty_like(m)
    for t in range(1, wl.T):
        a, b = vp.vp_shard_range(wl.V, wl.T, t)
        wt = dev_bf16(vp_inputs.make_weight_shard(wl, t))
        vp.vp_lmhead_ce_fwd(x_d, wt, y_d, a, b, m[t], s[t], zy[t])
        del wt
    logits = vp.vp_lmhead_logits(x_d, w0, lo, hi)
    vp.vp_logits_ce_stats(logits, y_d, lo, hi, None, m[0], s[0], zy[0])
    loss, lse, mean = vp.vp_ce_combine(m, s, zy, y_d)
    g = oracle.mean_scale(y)
    grads = vp.vp_logits_ce_bwd(logits, x_d, w0, y_d, lse, lo, hi, g)
    torch.cuda.synchronize()
    assert_loss_close(host(loss), gold["loss"])
    assert_loss_close(host(lse), gold["lse"], "lse")
    assert abs(float(mean.item()) - float(gold["mean"])) <= 2e-3
    x = vp_inputs.bf16_bits_to_f64(inp.x)
    w = vp_inputs.bf16_bits_to_f64(inp.w[lo:hi])
    r = np.random.default_rng(160)
    rows = r.choice(wl.N, 24, replace=False)
    err = float(np.abs(host(logits[torch.from_numpy(rows).cuda()])[:, :hi - lo]
                       - oracle.logits(x[rows], w)).max())
    log(f"  stored logits (24 rows): max abs err {err:.2e}")
    assert err <= 2e-3
    full_grads({"grads": {0: grads}}, 0, x, w, y, gold["lse"], lo, g)


def _sweep_cases():
    """Seeded shapes: odd N (1-2500), H a multiple of 8 (8-1024), Vs 1-5000 with T 1-4,
    so that stored rows are padded by 0-3 columns and the gradient GEMMs run as 128 x 128
    tiles or split over K; alternating one-read and two-pass statistics."""
    r = np.random.default_rng(4242)
    out = []
    for i in range(12):
        T = int(r.integers(1, 5))
        N = int(r.integers(1, 2501))
        H = 8 * int(r.integers(1, 129))
        Vs = int(r.integers(1, 5001))
        out.append((i, N, H, Vs, T, bool(i % 2)))
    return out


@pytest.mark.parametrize("case", _sweep_cases(),
                         ids=lambda c: f"{c[0]}-N{c[1]}-H{c[2]}-Vs{c[3]}-T{c[4]}-{'two' if c[5] else 'one'}")
def test_random_shape(vp, case):
    i, N, H, Vs, T, two_pass = case
    r = np.random.default_rng(5000 + i)
    V = Vs * T
    xb = vp_inputs.f32_to_bf16_bits(r.standard_normal((N, H)).astype(np.float32))
    wb = vp_inputs.f32_to_bf16_bits(
        r.standard_normal((V, H)).astype(np.float32) * np.float32(3.0 / math.sqrt(H)))
    y = r.integers(0, V, N).astype(np.int64)
    y[r.random(N) < 0.1] = -100
    _full_check(vp, xb, wb, y, T, two_pass, f"case {i}")
