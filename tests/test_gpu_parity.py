"""Parity of the HIP path with the fp64 oracle on the five workloads.

Every call goes through the C ABI (``vocab_lm_head_amd``), in the launch
configuration the benchmark times.  Small workloads are compared element by
element; at full size the oracle's per-token lse/loss come from
``tests/golden/oracle_<workload>.npz`` (written by
``tests/golden/make_oracle_golden.py``, which calls only the oracle), and
shard statistics, dX rows and dW rows are compared on seeded samples that the
oracle computes one by one.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import vp_inputs
from gpu_util import (assert_grad_close, assert_loss_close, assert_stats_close, bf16_bits,
                      dev_bf16, dev_i64, full_grads, host, log, run_ce_path)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def vp():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_lm_head_amd
    return vocab_lm_head_amd


def f64(bits):
    return vp_inputs.bf16_bits_to_f64(bits)


def _embed_case(vp, ids, w_bits, V, T, shards):
    """Bit-exact lookup of the given shards; returns the per-shard outputs."""
    ids_d = dev_i64(ids)
    w_d = dev_bf16(w_bits)
    outs = {}
    for t in shards:
        lo, hi = oracle.shard_range(V, T, t)
        got = bf16_bits(vp.vp_embed_fwd(ids_d, w_d[lo:hi], lo, hi))
        want = oracle.embed_shard(ids, w_bits[lo:hi], lo, hi)
        nbad = int((got != want).any(axis=1).sum())
        log(f"  embed shard {t}: {nbad} mismatching rows of {ids.size}")
        assert nbad == 0
        outs[t] = got
    return outs


# ---------------------------------------------------------------------------
def test_tiny_embedding_worked_example(vp):
    """V=8, T=2, ids [1, 6] -> [E1, 0] and [0, E6]; their sum is [E1, E6]."""
    inp = vp_inputs.make_inputs("tiny")
    wl = inp.wl
    outs = _embed_case(vp, inp.ids, inp.embed_w, wl.embed_V, wl.embed_T, range(wl.embed_T))
    assert np.array_equal(outs[0][0], inp.embed_w[1]) and not outs[0][1].any()
    assert np.array_equal(outs[1][1], inp.embed_w[6]) and not outs[1][0].any()
    # each id is owned by exactly one shard: the other's output is +0 bits, so OR == sum
    assert np.array_equal(outs[0] | outs[1], inp.embed_w[[1, 6]])


def test_tiny_ce(vp):
    """N=6, H=32, V=16, T=4: every shard, full comparison including the sum of dX partials."""
    inp = vp_inputs.make_inputs("tiny")
    wl = inp.wl
    x, w, y = f64(inp.x), f64(inp.w), inp.targets
    z = oracle.logits(x, w)
    loss, lse, mean = oracle.dense_ce(z, y)
    dz = oracle.dense_dlogits(z, y)
    dx, dw = oracle.shard_grads(x, w, dz)
    g = oracle.mean_scale(y)
    x_d, y_d, w_d = dev_bf16(inp.x), dev_i64(y), dev_bf16(inp.w)
    rng = [oracle.shard_range(wl.V, wl.T, t) for t in range(wl.T)]
    out = run_ce_path(vp, x_d, [w_d[a:b] for a, b in rng], [a for a, _ in rng],
                      [b for _, b in rng], y_d, g, bwd_shards=range(wl.T))
    for t, (a, b) in enumerate(rng):
        ref = oracle.shard_stats(z[:, a:b], y, a)
        assert_stats_close((host(out["m"][t]), host(out["s"][t]), host(out["zy"][t])), ref,
                           f"shard {t} stats")
    assert_loss_close(host(out["loss"]), loss)
    assert_loss_close(host(out["lse"]), lse, "lse")
    assert abs(float(out["mean"].item()) - mean) <= 2e-3
    dx_sum = sum(host(out["grads"][t][0]) for t in range(wl.T))
    assert_grad_close(dx_sum, dx, "dX (sum of shard partials)")
    for t, (a, b) in enumerate(rng):
        assert_grad_close(host(out["grads"][t][1]), dw[a:b], f"dW shard {t}")
        assert_grad_close(host(out["grads"][t][0]),
                          oracle.shard_grads(x, w[a:b], dz[:, a:b])[0], f"dX partial {t}")


def test_small_lm(vp):
    """N=4096, H=512, V=6400, T=2: both shards, full comparison; tied lookup of shard 0."""
    inp = vp_inputs.make_inputs("small_lm")
    wl = inp.wl
    _embed_case(vp, inp.ids, inp.w, wl.V, wl.T, [0, 1])
    x, w, y = f64(inp.x), f64(inp.w), inp.targets
    z = oracle.logits(x, w)
    loss, lse, mean = oracle.dense_ce(z, y)
    dz = oracle.dense_dlogits(z, y)
    g = oracle.mean_scale(y)
    x_d, y_d, w_d = dev_bf16(inp.x), dev_i64(y), dev_bf16(inp.w)
    rng = [oracle.shard_range(wl.V, wl.T, t) for t in range(wl.T)]
    out = run_ce_path(vp, x_d, [w_d[a:b] for a, b in rng], [a for a, _ in rng],
                      [b for _, b in rng], y_d, g, bwd_shards=[0, 1])
    for t, (a, b) in enumerate(rng):
        ref = oracle.shard_stats(z[:, a:b], y, a)
        assert_stats_close((host(out["m"][t]), host(out["s"][t]), host(out["zy"][t])), ref,
                           f"shard {t} stats")
    assert_loss_close(host(out["loss"]), loss)
    assert_loss_close(host(out["lse"]), lse, "lse")
    assert abs(float(out["mean"].item()) - mean) <= 2e-3
    for t, (a, b) in enumerate(rng):
        dxr, dwr = oracle.shard_grads(x, w[a:b], dz[:, a:b])
        assert_grad_close(host(out["grads"][t][0]), dxr, f"dX partial {t}")
        assert_grad_close(host(out["grads"][t][1]), dwr, f"dW shard {t}")


def _golden(name):
    path = os.path.join(GOLDEN, f"oracle_{name}.npz")
    if not os.path.exists(path):
        pytest.fail(f"{path} missing: run tests/golden/make_oracle_golden.py {name}")
    return np.load(path)


@pytest.mark.timeout(900)
def test_shard_8b(vp):
    """N=8192, H=4096, V=128256, T=8: all eight forwards, combine, backward of shards 0 and 7
    (their whole dX partials and dW against the oracle)."""
    inp = vp_inputs.make_inputs("shard_8b")
    wl = inp.wl
    gold = _golden("shard_8b")
    y = inp.targets
    g = oracle.mean_scale(y)
    x_d, y_d, w_d = dev_bf16(inp.x), dev_i64(y), dev_bf16(inp.w)
    rng = [oracle.shard_range(wl.V, wl.T, t) for t in range(wl.T)]
    log("  running 8 shard forwards, combine, 2 backwards")
    out = run_ce_path(vp, x_d, [w_d[a:b] for a, b in rng], [a for a, _ in rng],
                      [b for _, b in rng], y_d, g, bwd_shards=[0, 7])
    assert_loss_close(host(out["loss"]), gold["loss"])
    assert_loss_close(host(out["lse"]), gold["lse"], "lse")
    assert abs(float(out["mean"].item()) - float(gold["mean"])) <= 2e-3
    x = f64(inp.x)
    r = np.random.default_rng(100)
    sample = r.choice(wl.N, 64, replace=False)
    for t in (0, 7):
        a, b = rng[t]
        wt = f64(inp.w[a:b])
        ref = oracle.shard_stats(oracle.logits(x[sample], wt), y[sample], a)
        assert_stats_close((host(out["m"][t][sample]), host(out["s"][t][sample]),
                            host(out["zy"][t][sample])), ref, f"shard {t} stats (64 tokens)")
        full_grads(out, t, x, wt, y, gold["lse"], a, g)
    # tied lookup of shard 0 with Zipf ids
    _embed_case(vp, inp.ids, inp.w, wl.V, wl.T, [0, 5])


@pytest.mark.timeout(900)
def test_large_vocab(vp):
    """N=16384, H=8192, shard [19008, 8192] + 7 synthetic shards' statistics; shard 0's whole
    dX partial and dW against the oracle."""
    import torch
    inp = vp_inputs.make_inputs("large_vocab")
    wl = inp.wl
    gold = _golden("large_vocab")
    y = inp.targets
    g = oracle.mean_scale(y)
    ms, ss, zs = vp_inputs.synthetic_triples("large_vocab", y)
    x_d, y_d, w_d = dev_bf16(inp.x), dev_i64(y), dev_bf16(inp.w)
    Vs = wl.Vs
    starts = [t * Vs for t in range(wl.T)]
    ends = [(t + 1) * Vs for t in range(wl.T)]
    synth = {t: (torch.from_numpy(ms[t]).cuda(), torch.from_numpy(ss[t]).cuda(),
                 torch.from_numpy(zs[t]).cuda()) for t in range(1, wl.T)}
    shards = [w_d] + [None] * (wl.T - 1)
    out = run_ce_path(vp, x_d, shards, starts, ends, y_d, g, bwd_shards=[0], stats_rows=synth)
    assert_loss_close(host(out["loss"]), gold["loss"])
    assert_loss_close(host(out["lse"]), gold["lse"], "lse")
    assert abs(float(out["mean"].item()) - float(gold["mean"])) <= 2e-3
    x = f64(inp.x)
    w0 = f64(inp.w)
    r = np.random.default_rng(101)
    sample = r.choice(wl.N, 48, replace=False)
    ref = oracle.shard_stats(oracle.logits(x[sample], w0), y[sample], 0)
    assert_stats_close((host(out["m"][0][sample]), host(out["s"][0][sample]),
                        host(out["zy"][0][sample])), ref, "shard 0 stats (48 tokens)")
    full_grads(out, 0, x, w0, y, gold["lse"], 0, g)


def test_large_vocab_combine_synthetic(vp):
    """Standalone merge of 8 synthetic shards' statistics against the oracle's combine."""
    import torch
    wl = vp_inputs.WORKLOADS["large_vocab"]
    y = vp_inputs.make_inputs("large_vocab", with_weight=False).targets
    ms, ss, zs = vp_inputs.synthetic_triples("large_vocab", y)
    r = np.random.default_rng(7)   # row 0 is left to the caller: fill it like the others
    ms[0] = (3.6 + 0.3 * r.standard_normal(wl.N)).astype(np.float32)
    ss[0] = r.uniform(500, 1100, wl.N).astype(np.float32)
    own0 = (y // wl.Vs) == 0
    zs[0] = np.where(own0, ms[0] - r.uniform(0, 4, wl.N).astype(np.float32), 0).astype(np.float32)
    loss, lse, mean = oracle.combine_triples(ms.astype(np.float64), ss.astype(np.float64),
                                             zs.astype(np.float64), y)
    dl, dlse, dmean = vp.vp_ce_combine(torch.from_numpy(ms).cuda(), torch.from_numpy(ss).cuda(),
                                       torch.from_numpy(zs).cuda(), dev_i64(y))
    torch.cuda.synchronize()
    assert_loss_close(host(dl), loss)
    assert_loss_close(host(dlse), lse, "lse")
    assert abs(float(dmean.item()) - mean) <= 2e-3


@pytest.mark.timeout(900)
def test_embedding_heavy(vp):
    """Lookup of 65536 Zipf ids on shards 0 and 3 of [256000, 4096], then T=1 CE on 4096 tokens
    (the whole dX and dW against the oracle)."""
    inp = vp_inputs.make_inputs("embedding_heavy")
    wl = inp.wl
    _embed_case(vp, inp.ids, inp.w, wl.embed_V, wl.embed_T, [0, 3])
    gold = _golden("embedding_heavy")
    y = inp.targets
    g = oracle.mean_scale(y)
    x_d, y_d, w_d = dev_bf16(inp.x), dev_i64(y), dev_bf16(inp.w)
    out = run_ce_path(vp, x_d, [w_d], [0], [wl.V], y_d, g, bwd_shards=[0])
    assert_loss_close(host(out["loss"]), gold["loss"])
    assert_loss_close(host(out["lse"]), gold["lse"], "lse")
    assert abs(float(out["mean"].item()) - float(gold["mean"])) <= 2e-3
    x = f64(inp.x)
    w = f64(inp.w)
    r = np.random.default_rng(102)
    sample = r.choice(wl.N, 32, replace=False)
    ref = oracle.shard_stats(oracle.logits(x[sample], w), y[sample], 0)
    assert_stats_close((host(out["m"][0][sample]), host(out["s"][0][sample]),
                        host(out["zy"][0][sample])), ref, "stats (32 tokens)")
    full_grads(out, 0, x, w, y, gold["lse"], 0, g)
