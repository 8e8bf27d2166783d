"""Weight gradient of the masked lookup (vp_embed_bwd) against the oracle's
scatter-add, through the C ABI binding.

Tolerance, derived from the arithmetic: each element of the result is dw0 plus an
fp32 sum of the bf16 gradient values of the L tokens that own the row (exact in
fp32 once widened), so in any summation order

    |gpu - exact| <= (L + 1) * 2^-24 * (sum |x| + |dw0|)

(the standard bound for recursive summation, with one more rounding for the
addition to dw0).  That is far tighter than the 1e-2 relative bar of the LM-head
gradients and fails on a single dropped or doubled token; the 1e-2 bar is
checked too.  Rows that no owned id names must come back bit-for-bit unchanged.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import vp_inputs
from gpu_util import (U, dev_bf16, dev_i64, embed_bwd_full_check,
                      embed_bwd_run, host, log)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vp():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_lm_head_amd
    return vocab_lm_head_amd


def _dout(seed, n, h, scale=1.0):
    r = np.random.default_rng(seed)
    return vp_inputs.f32_to_bf16_bits(r.standard_normal((n, h)).astype(np.float32) * scale)


def test_worked_example_backwards(vp):
    """V=8, T=2, ids [1, 6]: token 0's gradient is shard 0's row 1, token 1's is shard 1's
    row 2, bit for bit; every other row stays zero."""
    inp = vp_inputs.make_inputs("tiny")
    wl = inp.wl
    dout = _dout(0, 2, wl.embed_H)
    for t in range(wl.embed_T):
        lo, hi = vp.vp_shard_range(wl.embed_V, wl.embed_T, t)
        got = host(embed_bwd_run(vp, inp.ids, dout, lo, hi, np.zeros((hi - lo, wl.embed_H), np.float32)))
        want = oracle.embed_shard_grad(inp.ids, vp_inputs.bf16_bits_to_f64(dout), lo, hi)
        assert np.array_equal(got, want), t


def test_small_lm_tied_ids(vp):
    """4096 uniform ids over V=6400 (T=2, H=512), both shards, every row."""
    inp = vp_inputs.make_inputs("small_lm", with_weight=False)
    wl = inp.wl
    dout = vp_inputs.make_embed_output_grad("small_lm")
    for t in range(wl.embed_T):
        lo, hi = vp.vp_shard_range(wl.embed_V, wl.embed_T, t)
        embed_bwd_full_check(vp, inp.ids, dout, lo, hi, label=f"small_lm shard {t}")


def test_accumulates_and_is_deterministic(vp):
    """The gradient is added to dw (here a random prefill), and two calls on the same
    inputs give the same bits."""
    r = np.random.default_rng(5)
    n, h, lo, hi = 3000, 264, 1000, 1700
    ids = np.minimum(r.zipf(1.2, n) + 990, 2000).astype(np.int64)
    dout = _dout(6, n, h)
    dw0 = r.standard_normal((hi - lo, h)).astype(np.float32)
    a = embed_bwd_full_check(vp, ids, dout, lo, hi, dw0, "prefilled, Zipf ids")
    b = host(embed_bwd_run(vp, ids, dout, lo, hi, dw0))
    assert np.array_equal(a, b), "two calls differ"


EDGE_CASES = ["all_off_shard", "one_long_row", "shard_edges", "single_token",
              "three_passes_ragged_cols", "wide_row_two_col_blocks"]


@pytest.mark.parametrize("case", EDGE_CASES)
def test_edges(vp, case):
    r = np.random.default_rng(40 + EDGE_CASES.index(case))
    if case == "all_off_shard":
        n, h, lo, hi = 700, 64, 100, 200
        ids = np.concatenate([r.integers(-50, 100, n // 2), r.integers(200, 400, n - n // 2)])
    elif case == "one_long_row":        # one row, 5000 tokens: crosses many blocks and two sort tiles
        n, h, lo, hi = 5000, 128, 0, 64
        ids = np.full(n, 37, dtype=np.int64)
    elif case == "shard_edges":
        n, h, lo, hi = 900, 40, 512, 1024
        edge = np.array([512, 1023, 1024, 511, -1, -100, 4096, 2**40, -2**40], dtype=np.int64)
        ids = edge[r.integers(0, edge.size, n)]
    elif case == "single_token":
        n, h, lo, hi = 1, 16, 0, 10
        ids = np.array([9], dtype=np.int64)
    elif case == "three_passes_ragged_cols":   # Vs = 70000 needs 17-bit keys: three 8-bit passes
        n, h, lo, hi = 9000, 8, 0, 70000
        ids = np.concatenate([r.integers(-10, 70010, n - 2000), np.full(2000, 69999)])
        r.shuffle(ids)
    else:                                      # h = 2056: a full and a ragged column block
        n, h, lo, hi = 1200, 2056, 300, 420
        ids = r.integers(280, 440, n)
    ids = np.asarray(ids, dtype=np.int64)
    dout = _dout(7, n, h)
    dw0 = r.standard_normal((hi - lo, h)).astype(np.float32)
    log(f"  case {case}: n={n} h={h} rows={hi - lo}")
    embed_bwd_full_check(vp, ids, dout, lo, hi, dw0, case)


@pytest.mark.timeout(900)
def test_embedding_heavy_backward(vp):
    """65536 Zipf(1.0) ids on shard 0 ([64000, 4096] of V=256000, T=4), added into a random
    prefilled gradient (the tied shard's LM-head gradient): every row of the shard against the
    oracle's scatter-add within the summation bound (rows no id names unchanged bit for bit),
    plus every column's total over the shard against the owned tokens' total."""
    import torch
    inp = vp_inputs.make_inputs("embedding_heavy", with_weight=False)
    wl = inp.wl
    lo, hi = vp.vp_shard_range(wl.embed_V, wl.embed_T, 0)
    ids = inp.ids
    dout = vp_inputs.make_embed_output_grad("embedding_heavy")
    own = (ids >= lo) & (ids < hi)
    rows, counts = np.unique(ids[own] - lo, return_counts=True)
    log(f"  {own.sum()} owned ids, {rows.size} distinct rows, most repeated row x{counts.max()}")
    dw0 = (np.random.default_rng(8).standard_normal((hi - lo, wl.embed_H), dtype=np.float32)
           * np.float32(1e-3))
    got = embed_bwd_full_check(vp, ids, dout, lo, hi, dw0, "embedding-heavy, every row")
    dout_f = vp_inputs.bf16_bits_to_f64(dout[own])
    col_gpu = (got - dw0.astype(np.float64)).sum(axis=0)
    col_ref = dout_f.sum(axis=0)
    mag = np.abs(dout_f).sum(axis=0) + np.abs(dw0).astype(np.float64).sum(axis=0)
    err = np.abs(col_gpu - col_ref)
    log(f"  column totals: max abs err {err.max():.3e}")
    assert np.all(err <= (own.sum() + 2) * U * mag * 2 + 1e-9)
