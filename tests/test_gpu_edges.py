"""Edge cases of the HIP path against the oracle: ragged tiles, ignore_index,
degenerate shards, closed forms, empty inputs and lookup boundaries.  All go
through the C ABI binding."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import vp_inputs
from gpu_util import (assert_grad_close, assert_loss_close, assert_stats_close, bf16_bits,
                      dev_bf16, dev_i64, host, log, run_ce_path)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vp():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_lm_head_amd
    return vocab_lm_head_amd


def _problem(seed, N, H, V, x_std=1.0, logit_std=3.0, ignore_frac=0.0):
    r = np.random.default_rng(seed)
    xb = vp_inputs.f32_to_bf16_bits(r.standard_normal((N, H)).astype(np.float32) * x_std)
    wb = vp_inputs.f32_to_bf16_bits(
        r.standard_normal((V, H)).astype(np.float32) * (logit_std / math.sqrt(H) / x_std))
    y = r.integers(0, V, N).astype(np.int64)
    if ignore_frac:
        y[r.random(N) < ignore_frac] = -100
    return xb, wb, y


def _full_check(vp, xb, wb, y, T, bwd_shards=None, label=""):
    N, H = xb.shape
    V = wb.shape[0]
    x, w = vp_inputs.bf16_bits_to_f64(xb), vp_inputs.bf16_bits_to_f64(wb)
    z = oracle.logits(x, w)
    loss, lse, mean = oracle.dense_ce(z, y)
    dz = oracle.dense_dlogits(z, y)
    g = oracle.mean_scale(y)
    rng = [oracle.shard_range(V, T, t) for t in range(T)]
    x_d, w_d, y_d = dev_bf16(xb), dev_bf16(wb), dev_i64(y)
    bwd = list(range(T)) if bwd_shards is None else bwd_shards
    log(f"  case {label}: N={N} H={H} V={V} T={T}")
    out = run_ce_path(vp, x_d, [w_d[a:b] for a, b in rng], [a for a, _ in rng],
                      [b for _, b in rng], y_d, g, bwd_shards=bwd)
    for t, (a, b) in enumerate(rng):
        assert_stats_close((host(out["m"][t]), host(out["s"][t]), host(out["zy"][t])),
                           oracle.shard_stats(z[:, a:b], y, a), f"shard {t} stats")
    assert_loss_close(host(out["loss"]), loss)
    assert_loss_close(host(out["lse"]), lse, "lse")
    assert abs(float(out["mean"].item()) - mean) <= 2e-3
    for t in bwd:
        a, b = rng[t]
        dxr, dwr = oracle.shard_grads(x, w[a:b], dz[:, a:b])
        assert_grad_close(host(out["grads"][t][0]), dxr, f"dX partial {t}")
        assert_grad_close(host(out["grads"][t][1]), dwr, f"dW {t}")
    return out


def test_ragged_tiles(vp):
    """N, Vs and H all off the 256 / 64 tile grid: 300 tokens, 3 shards of 700, H = 136."""
    xb, wb, y = _problem(1, 300, 136, 2100)
    _full_check(vp, xb, wb, y, T=3, label="ragged")


def test_ignore_index(vp):
    xb, wb, y = _problem(2, 257, 64, 1024, ignore_frac=0.3)
    out = _full_check(vp, xb, wb, y, T=2, label="ignore_index 30%")
    ign = y == -100
    assert not host(out["loss"])[ign].any()
    for t in out["grads"]:
        assert not host(out["grads"][t][0])[ign].any(), "ignored tokens must get dX = 0"


def test_ignore_index_inside_the_vocabulary(vp):
    """ignore_index = 517, a real id of shard 1 (V = 1024, T = 2): every 7th token targets it
    and is ignored -- loss 0, no gradient, left out of the mean -- although each shard's
    forward still picks its logit as that token's target (the statistics do not know which
    id is ignored)."""
    xb, wb, y = _problem(9, 300, 64, 1024)
    ign = 517
    y[::7] = ign
    N, H = xb.shape
    V, T = wb.shape[0], 2
    x, w = vp_inputs.bf16_bits_to_f64(xb), vp_inputs.bf16_bits_to_f64(wb)
    z = oracle.logits(x, w)
    loss, lse, mean = oracle.dense_ce(z, y, ignore_index=ign)
    dz = oracle.dense_dlogits(z, y, ignore_index=ign)
    g = oracle.mean_scale(y, ign)
    rng = [oracle.shard_range(V, T, t) for t in range(T)]
    x_d, w_d, y_d = dev_bf16(xb), dev_bf16(wb), dev_i64(y)
    out = run_ce_path(vp, x_d, [w_d[a:b] for a, b in rng], [a for a, _ in rng],
                      [b for _, b in rng], y_d, g, bwd_shards=[0, 1], ignore_index=ign)
    for t, (a, b) in enumerate(rng):
        assert_stats_close((host(out["m"][t]), host(out["s"][t]), host(out["zy"][t])),
                           oracle.shard_stats(z[:, a:b], y, a), f"shard {t} stats")
    assert_loss_close(host(out["loss"]), loss)
    assert not host(out["loss"])[y == ign].any()
    assert abs(float(out["mean"].item()) - mean) <= 2e-3
    for t, (a, b) in enumerate(rng):
        dxr, dwr = oracle.shard_grads(x, w[a:b], dz[:, a:b])
        assert_grad_close(host(out["grads"][t][0]), dxr, f"dX partial {t}")
        assert_grad_close(host(out["grads"][t][1]), dwr, f"dW {t}")
        assert not host(out["grads"][t][0])[y == ign].any(), "ignored tokens must get dX = 0"


def test_out_of_range_targets_follow_the_contract(vp):
    """Targets outside [0, V) that are not ignore_index (V + 5, -7, 2^40) break the data
    contract; the header defines what the GPU then does: such a target is off-shard on every
    shard, so no shard picks a target logit (loss = lse), the token still counts in the mean,
    and its gradient has no onehot term.  Expected values: the oracle on the same tokens with
    those targets replaced by 0, then the onehot that replacement subtracted added back."""
    xb, wb, y = _problem(11, 64, 64, 600)
    bad = np.array([0, 1, 2])
    y[bad] = [600 + 5, -7, 2**40]
    N, V, T = 64, 600, 3
    x, w = vp_inputs.bf16_bits_to_f64(xb), vp_inputs.bf16_bits_to_f64(wb)
    z = oracle.logits(x, w)
    y_rep = y.copy()
    y_rep[bad] = 0
    loss, lse, _ = oracle.dense_ce(z, y_rep)
    loss[bad] = lse[bad]
    mean = loss.sum() / N
    g = oracle.mean_scale(y)                        # all 64 tokens count
    dz = oracle.dense_dlogits(z, y_rep, scale=g)
    dz[bad, 0] += g
    rng = [oracle.shard_range(V, T, t) for t in range(T)]
    x_d, w_d, y_d = dev_bf16(xb), dev_bf16(wb), dev_i64(y)
    out = run_ce_path(vp, x_d, [w_d[a:b] for a, b in rng], [a for a, _ in rng],
                      [b for _, b in rng], y_d, g, bwd_shards=range(T))
    assert_loss_close(host(out["loss"]), loss)
    assert_loss_close(host(out["lse"]), lse, "lse")
    assert abs(float(out["mean"].item()) - mean) <= 2e-3
    for t, (a, b) in enumerate(rng):
        dxr, dwr = oracle.shard_grads(x, w[a:b], dz[:, a:b])
        assert_grad_close(host(out["grads"][t][0]), dxr, f"dX partial {t}")
        assert_grad_close(host(out["grads"][t][1]), dwr, f"dW {t}")


def test_all_ignored(vp):
    """N_valid = 0: mean 0 (max(1, N_valid) guard), loss 0, every gradient 0."""
    xb, wb, y = _problem(3, 40, 32, 96)
    y[:] = -100
    out = _full_check(vp, xb, wb, y, T=2, label="all ignored")
    assert float(out["mean"].item()) == 0.0
    for t in out["grads"]:
        assert not host(out["grads"][t][0]).any() and not host(out["grads"][t][1]).any()


def test_degenerate_one_row_shards(vp):
    """Vs = 1 (V = T = 4), one token, H = 8 (a single partial K step)."""
    xb, wb, y = _problem(4, 1, 8, 4)
    _full_check(vp, xb, wb, y, T=4, label="Vs=1")
    xb, wb, y = _problem(5, 3, 8, 4)
    _full_check(vp, xb, wb, y, T=1, label="T=1, V=4")


def test_targets_on_shard_edges(vp):
    N, H, V, T = 64, 96, 512, 4
    xb, wb, _ = _problem(6, N, H, V)
    Vs = V // T
    edges = np.array([t * Vs + d for t in range(T) for d in (0, Vs - 1)], dtype=np.int64)
    y = np.resize(edges, N)
    _full_check(vp, xb, wb, y, T=T, label="edge targets")


@pytest.mark.parametrize("T", [9, 16, 17, 33])
def test_combine_many_shards(vp, T):
    """Combine over more shards than it reads in one batch (8): per-shard statistics
    of a dense problem (fp32, as the forward hands them over), merged on the GPU,
    against the dense loss of the same logits; 20% of the targets are ignored."""
    import torch
    r = np.random.default_rng(100 + T)
    N, Vs = 300, 7
    V = T * Vs
    z = r.standard_normal((N, V)) * 4.0 + r.standard_normal((1, V)) * 3.0
    y = r.integers(0, V, N).astype(np.int64)
    y[r.random(N) < 0.2] = -100
    stats = [oracle.shard_stats(z[:, t * Vs:(t + 1) * Vs], y, t * Vs) for t in range(T)]
    m, s, zy = (np.stack([st[k] for st in stats]).astype(np.float32) for k in range(3))
    loss, lse, mean = oracle.dense_ce(z, y)
    log(f"  combine T={T}, N={N}")
    dl, dlse, dmean = vp.vp_ce_combine(torch.from_numpy(m).cuda(), torch.from_numpy(s).cuda(),
                                       torch.from_numpy(zy).cuda(), dev_i64(y))
    torch.cuda.synchronize()
    assert_loss_close(host(dl), loss)
    assert_loss_close(host(dlse), lse, "lse")
    assert abs(float(dmean.item()) - mean) <= 2e-3


def test_combine_extreme_spreads(vp):
    """Shard maxima up to 200 apart, so the far shards' rescaled sums underflow to nothing,
    sums from 1 to Vs, and targets owned by shards far below the global maximum (losses
    near 200); 10% ignored.  The merge against the oracle's combine in fp64 of the same
    fp32 statistics."""
    import torch
    r = np.random.default_rng(55)
    T, N, Vs = 8, 2000, 20000
    m = r.uniform(-100.0, 100.0, (T, N))
    s = np.exp(r.uniform(0.0, np.log(Vs), (T, N)))
    owner = r.integers(0, T, N)
    y = (owner * Vs + r.integers(0, Vs, N)).astype(np.int64)
    y[r.random(N) < 0.1] = -100
    zy = np.zeros((T, N))
    zy[owner, np.arange(N)] = m[owner, np.arange(N)] - r.uniform(0.0, 40.0, N)
    m, s, zy = (a.astype(np.float32) for a in (m, s, zy))
    loss, lse, mean = oracle.combine_triples(m.astype(np.float64), s.astype(np.float64),
                                             zy.astype(np.float64), y)
    log(f"  losses up to {loss.max():.1f}")
    dl, dlse, dmean = vp.vp_ce_combine(torch.from_numpy(m).cuda(), torch.from_numpy(s).cuda(),
                                       torch.from_numpy(zy).cuda(), dev_i64(y))
    torch.cuda.synchronize()
    assert_loss_close(host(dl), loss)
    assert_loss_close(host(dlse), lse, "lse")
    assert abs(float(dmean.item()) - mean) <= 2e-3


def test_twelve_shards_full_path(vp):
    """T=12 (V=1200, Vs=100): every shard's forward, combine over 12, backward of three shards."""
    xb, wb, y = _problem(12, 333, 64, 1200, logit_std=4.0, ignore_frac=0.1)
    _full_check(vp, xb, wb, y, T=12, bwd_shards=[0, 5, 11], label="T=12")


@pytest.mark.parametrize("pad_rows", ["random", "zero"])
def test_padded_vocabulary(vp, pad_rows):
    """The pages' padding example: GPT-2's V = 50257 padded to 51200 for T = 8 (each shard
    6400 = 50 x 128 rows).  The extra rows are ordinary rows no target uses (random or zero
    weights); the whole path runs on V_pad and matches the oracle's dense CE over V_pad."""
    V, T = 50257, 8
    V_pad = vp.vp_padded_vocab(V, T, 128)
    assert V_pad == 51200
    r = np.random.default_rng(50257)
    N, H = 300, 64
    xb = vp_inputs.f32_to_bf16_bits(r.standard_normal((N, H)).astype(np.float32))
    w = r.standard_normal((V_pad, H)).astype(np.float32) * (3.0 / math.sqrt(H))
    if pad_rows == "zero":
        w[V:] = 0.0
    wb = vp_inputs.f32_to_bf16_bits(w)
    y = r.integers(0, V, N).astype(np.int64)
    y[:8] = V - 1                        # the last real id, in the shard holding the padding
    _full_check(vp, xb, wb, y, T=T, bwd_shards=[0, 7], label=f"V_pad=51200 ({pad_rows} padding)")


@pytest.mark.parametrize("shape", [(1, 64, 40, 2), (257, 64, 514, 2), (255, 8, 255, 1)])
def test_tile_boundaries(vp, shape):
    """A single token, and sizes one past / one short of a 256-row tile in both the token
    and the vocabulary dimension (N, H, V, T), H down to 8."""
    N, H, V, T = shape
    xb, wb, y = _problem(1000 + N, N, H, V, logit_std=3.0)
    _full_check(vp, xb, wb, y, T=T, label=f"N={N} H={H} V={V}")


def test_deterministic(vp):
    """The forward, combine and backward use no atomics: two calls on the same inputs give
    the same bits (statistics, loss, lse, mean, dX, dW)."""
    import torch
    xb, wb, y = _problem(77, 700, 136, 1200, logit_std=4.0, ignore_frac=0.1)
    x_d, w_d, y_d = dev_bf16(xb), dev_bf16(wb), dev_i64(y)
    rng = [oracle.shard_range(1200, 3, t) for t in range(3)]
    g = oracle.mean_scale(y)
    runs = [run_ce_path(vp, x_d, [w_d[a:b] for a, b in rng], [a for a, _ in rng],
                        [b for _, b in rng], y_d, g, bwd_shards=[0, 2]) for _ in range(2)]
    for key in ("m", "s", "zy", "loss", "lse", "mean"):
        assert torch.equal(runs[0][key], runs[1][key]), key
    for t in (0, 2):
        for k in range(2):
            assert torch.equal(runs[0]["grads"][t][k], runs[1]["grads"][t][k]), (t, k)


@pytest.mark.parametrize("shape", [(8192, 4096, 16032), (4096, 512, 3200)],
                         ids=["shard_8b", "small_lm"])
def test_deterministic_at_full_size(vp, shape):
    """The GEMMs order their LDS traffic with explicit waits and barriers; a missing wait
    would show as run-to-run differences under full load.  Three runs of the forward,
    combine (T = 1) and backward on the same inputs must give the same bits: at the
    8B-class shard (2016, 512 and 1008 tiles) and at the small LM, whose two gradient GEMMs
    run as 128 x 128 tiles in one launch."""
    import torch
    N, H, Vs = shape
    g = torch.Generator(device="cuda").manual_seed(N + H)
    x = torch.randn((N, H), device="cuda", generator=g).bfloat16()
    w = (0.02 * torch.randn((Vs, H), device="cuda", generator=g)).bfloat16()
    y = torch.randint(0, 8 * Vs, (N,), device="cuda", generator=g)
    y[::13] = -100
    log(f"  N={N} H={H} Vs={Vs}: three runs")
    runs = []
    for _ in range(3):
        m, s, zy = vp.vp_lmhead_ce_fwd(x, w, y, 0, Vs)
        loss, lse, mean = vp.vp_ce_combine(m[None], s[None], zy[None], y)
        dx, dw = vp.vp_lmhead_ce_bwd(x, w, y, lse, 0, Vs, 1.0 / N)
        torch.cuda.synchronize()
        runs.append((m, s, zy, loss, lse, mean, dx, dw))
    names = ("m", "s", "zy", "loss", "lse", "mean", "dx", "dw")
    for r in runs[1:]:
        for name, a, b in zip(names, runs[0], r):
            assert torch.equal(a, b), f"{name} differs between runs"
    assert bool(torch.isfinite(runs[0][6]).all()) and bool(torch.isfinite(runs[0][7]).all())


@pytest.mark.parametrize("scale", [1.0, 0.0, -0.25, 4096.0])
def test_grad_scale_other_than_the_mean(vp, scale):
    """grad_scale is the caller's upstream factor: 1 for a summed loss, 0, a negative one,
    and a loss-scaling factor.  dX and dW follow the oracle's dlogits at that factor, and
    at 0 both are exactly zero."""
    xb, wb, y = _problem(91, 300, 136, 1400, ignore_frac=0.1)
    x, w = vp_inputs.bf16_bits_to_f64(xb), vp_inputs.bf16_bits_to_f64(wb)
    z = oracle.logits(x, w)
    dz = oracle.dense_dlogits(z, y, scale=scale)
    rng = [oracle.shard_range(1400, 2, t) for t in range(2)]
    x_d, w_d, y_d = dev_bf16(xb), dev_bf16(wb), dev_i64(y)
    log(f"  grad_scale {scale}")
    out = run_ce_path(vp, x_d, [w_d[a:b] for a, b in rng], [a for a, _ in rng],
                      [b for _, b in rng], y_d, scale, bwd_shards=[0, 1])
    for t, (a, b) in enumerate(rng):
        dxr, dwr = oracle.shard_grads(x, w[a:b], dz[:, a:b])
        dx, dw = host(out["grads"][t][0]), host(out["grads"][t][1])
        if scale == 0.0:
            assert not dx.any() and not dw.any(), "grad_scale 0 must give zero gradients"
        else:
            assert_grad_close(dx, dxr, f"dX partial {t}")
            assert_grad_close(dw, dwr, f"dW {t}")


def test_large_logits(vp):
    """Logit std 40: the stabilising maximum matters; sum-exp must not overflow."""
    xb, wb, y = _problem(7, 130, 128, 640, logit_std=40.0)
    _full_check(vp, xb, wb, y, T=2, label="logit std 40")


def test_uniform_logits_closed_form(vp):
    """W = 0 -> every logit equal -> loss = log V exactly, at the 8B-class shard shape."""
    import json
    import os
    import torch
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ce_closed_forms.json")))
    V = 128256
    want = [c["loss"] for c in gold["uniform"]["cases"] if c["V"] == V][0]
    N, H, T = 512, 4096, 8
    r = np.random.default_rng(8)
    x_d = dev_bf16(vp_inputs.f32_to_bf16_bits(r.standard_normal((N, H)).astype(np.float32)))
    w_d = torch.zeros((V // T, H), dtype=torch.bfloat16, device="cuda")
    y = r.integers(0, V, N).astype(np.int64)
    y_d = dev_i64(y)
    rng = [oracle.shard_range(V, T, t) for t in range(T)]
    out = run_ce_path(vp, x_d, [w_d] * T, [a for a, _ in rng], [b for _, b in rng], y_d,
                      1.0 / N, bwd_shards=[0])
    loss = host(out["loss"])
    log(f"  uniform: loss range [{loss.min():.7f}, {loss.max():.7f}] vs log V = {want:.7f}")
    assert np.abs(loss - want).max() <= 2e-3
    # gradient closed form: dz = (1/V - [j == y]) / N, so dW_0[j] = (X^T (1/V - onehot_j)) / N
    x = vp_inputs.bf16_bits_to_f64(bf16_bits(x_d))
    Vs = V // T
    onehot = (y[:, None] == np.arange(Vs)[None, :]).astype(np.float64)
    dz0 = (1.0 / V - onehot) / N
    assert_grad_close(host(out["grads"][0][1]), dz0.T @ x, "dW_0 closed form")
    assert not host(out["grads"][0][0]).any(), "dX_0 = dz_0 W_0 = 0 when W_0 = 0"


def test_empty_inputs(vp):
    import torch
    d = "cuda"
    x = torch.empty((0, 16), dtype=torch.bfloat16, device=d)
    w = torch.zeros((8, 16), dtype=torch.bfloat16, device=d)
    y = torch.empty(0, dtype=torch.int64, device=d)
    out = vp.vp_embed_fwd(y, w, 0, 8)
    assert out.shape == (0, 16)
    m, s, zy = vp.vp_lmhead_ce_fwd(x, w, y, 0, 8)
    assert m.shape == (0,)
    st = torch.empty((2, 0), dtype=torch.float32, device=d)
    loss, lse, mean = vp.vp_ce_combine(st, st, st, y)
    lse_in = torch.empty(0, dtype=torch.float32, device=d)
    dw = torch.full((8, 16), 7.0, dtype=torch.float32, device=d)
    dx, dw = vp.vp_lmhead_ce_bwd(x, w, y, lse_in, 0, 8, 1.0, dw=dw)
    torch.cuda.synchronize()
    assert float(mean.item()) == 0.0
    assert not dw.any().item(), "no tokens -> dW = 0"


def test_embedding_boundaries(vp):
    V, T, H = 4096, 4, 8
    r = np.random.default_rng(9)
    wb = r.integers(0, 65536, (V, H)).astype(np.uint16)
    Vs = V // T
    ids = np.concatenate([[-1, -100, V, V + 5, 2**40, -(2**40)],
                          [t * Vs + d for t in range(T) for d in (-1, 0, 1, Vs - 1)],
                          r.integers(-10, V + 10, 1000)]).astype(np.int64)
    w_d, ids_d = dev_bf16(wb), dev_i64(ids)
    total = np.zeros((ids.size, H), dtype=np.uint64)
    for t in range(T):
        lo, hi = oracle.shard_range(V, T, t)
        got = bf16_bits(vp.vp_embed_fwd(ids_d, w_d[lo:hi], lo, hi))
        want = oracle.embed_shard(ids, wb[lo:hi], lo, hi)
        assert np.array_equal(got, want), f"shard {t}"
        total += got
    inr = (ids >= 0) & (ids < V)
    assert np.array_equal(total[inr].astype(np.uint16), wb[ids[inr]])
    assert not total[~inr].any()


def test_embedding_wide_rows(vp):
    """H = 8200 (not a multiple of the 4 x 64 x 8 unrolled row step), odd N."""
    V, T, H = 300, 3, 8200
    r = np.random.default_rng(10)
    wb = r.integers(0, 65536, (V, H)).astype(np.uint16)
    ids = r.integers(-3, V + 3, 777).astype(np.int64)
    w_d, ids_d = dev_bf16(wb), dev_i64(ids)
    for t in range(T):
        lo, hi = oracle.shard_range(V, T, t)
        got = bf16_bits(vp.vp_embed_fwd(ids_d, w_d[lo:hi], lo, hi))
        assert np.array_equal(got, oracle.embed_shard(ids, wb[lo:hi], lo, hi))


def test_invalid_arguments_raise(vp):
    import torch
    d = "cuda"
    x = torch.zeros((4, 12), dtype=torch.bfloat16, device=d)   # H % 8 != 0
    w = torch.zeros((8, 12), dtype=torch.bfloat16, device=d)
    y = torch.zeros(4, dtype=torch.int64, device=d)
    with pytest.raises(vp.VPError) as e:
        vp.vp_lmhead_ce_fwd(x, w, y, 0, 8)
    assert e.value.status == -4
    with pytest.raises(vp.VPError):
        vp.vp_shard_range(10, 4, 0)


def test_binding_rejects_mismatched_buffers(vp):
    """The binding refuses caller buffers the kernels would overrun or could not address,
    before anything is launched: short outputs, a host workspace, an undersized one."""
    import torch
    d = "cuda"
    n, h, vs = 64, 16, 40
    x = torch.zeros((n, h), dtype=torch.bfloat16, device=d)
    w = torch.zeros((vs, h), dtype=torch.bfloat16, device=d)
    y = torch.zeros(n, dtype=torch.int64, device=d)
    lse = torch.zeros(n, dtype=torch.float32, device=d)
    f32 = lambda *s: torch.zeros(s, dtype=torch.float32, device=d)
    with pytest.raises(ValueError):
        vp.vp_lmhead_ce_bwd(x, w, y, lse, 0, vs, 1.0, dx=f32(n - 1, h))
    with pytest.raises(ValueError):
        vp.vp_lmhead_ce_bwd(x, w, y, lse, 0, vs, 1.0, dw=f32(vs, h - 8))
    with pytest.raises(ValueError):
        vp.vp_lmhead_ce_bwd(x, w, y, lse, 0, vs, 1.0,
                            workspace=torch.zeros(1 << 20, dtype=torch.uint8))
    with pytest.raises(vp.VPError) as e:
        vp.vp_lmhead_ce_bwd(x, w, y, lse, 0, vs, 1.0,
                            workspace=torch.zeros(64, dtype=torch.uint8, device=d))
    assert e.value.status == -5
    with pytest.raises(ValueError):
        vp.vp_lmhead_ce_fwd(x, w, y, 0, vs, m_local=f32(n // 2))
    logits = vp.vp_lmhead_logits(x, w, 0, vs)
    with pytest.raises(ValueError):
        vp.vp_logits_ce_stats(logits, y, 0, vs, s_local=f32(n + 1))
    with pytest.raises(ValueError):
        vp.vp_logits_ce_bwd(logits, x, w, y, lse, 0, vs, 1.0, dx=f32(n, h + 8))
    with pytest.raises(ValueError):
        vp.vp_logits_ce_bwd(logits, x, w, y[: n - 1], lse, 0, vs, 1.0)
    with pytest.raises(ValueError):
        vp.vp_ce_max(f32(2, n), out=f32(n - 1))
    with pytest.raises(ValueError):
        vp.vp_embed_bwd(y, x, 0, vs, workspace=torch.zeros(1 << 20, dtype=torch.uint8))
    torch.cuda.synchronize()
