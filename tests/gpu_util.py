"""Helpers of the GPU parity tests: moving input bits to the device, running the
HIP path through the C ABI binding, and the comparison bars.

Tolerances (floating point):
  per-token loss and lse     max abs error <= 2e-3
  dX, dW                     max|gpu - oracle| / max|oracle| <= 1e-2 per tensor
  shard statistics m, zy     max abs error <= 2e-3;  s: max relative error <= 2e-3
Integer / byte work (the embedding) is compared bit for bit.

The lookup gradient: each element is dw0 plus an fp32 sum of the bf16 gradient values
of the L tokens that own the row (exact in fp32 once widened), so in any summation
order |gpu - exact| <= (L + 1) 2^-24 (sum |x| + |dw0|), the recursive-summation bound
with one more rounding for the addition to dw0.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import vp_inputs

LOSS_ATOL = 2e-3
GRAD_RTOL = 1e-2
STAT_ATOL = 2e-3
STAT_RTOL = 2e-3
U = 2.0 ** -24       # fp32 unit roundoff


def log(msg: str) -> None:
    print(msg, flush=True)


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def dev_i64(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float64)


def rel_max(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.abs(b).max()
    num = np.abs(a - b).max()
    return float(num / den) if den > 0 else float(num)


def assert_loss_close(gpu, ref, what="loss"):
    err = float(np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64)).max())
    log(f"  {what}: max abs err {err:.3e} (bar {LOSS_ATOL})")
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    assert err <= LOSS_ATOL, f"{what}: max abs err {err} > {LOSS_ATOL}"


def assert_grad_close(gpu, ref, what):
    e = rel_max(gpu, ref)
    log(f"  {what}: max|d|/max|ref| {e:.3e} (bar {GRAD_RTOL})")
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    assert e <= GRAD_RTOL, f"{what}: relative error {e} > {GRAD_RTOL}"


def assert_stats_close(gpu, ref, what="stats"):
    (gm, gs, gz), (rm, rs, rz) = gpu, ref
    em = float(np.abs(gm - rm).max())
    ez = float(np.abs(gz - rz).max())
    es = float((np.abs(gs - rs) / np.abs(rs)).max())
    log(f"  {what}: m {em:.2e}  s(rel) {es:.2e}  zy {ez:.2e}")
    assert em <= STAT_ATOL and ez <= STAT_ATOL and es <= STAT_RTOL, (em, es, ez)


def run_ce_path(vp, x_d, w_shards_d, starts, ends, tgt_d, grad_scale, bwd_shards,
                ignore_index=-100, stats_rows=None):
    """All shards' forwards -> combine -> selected shards' backwards, on the GPU.

    Returns dict with loss, lse, mean (device tensors), the stacked statistics
    [T, n], and {shard: (dx, dw)} for ``bwd_shards``.
    """
    n = x_d.shape[0]
    T = len(w_shards_d)
    m = torch.empty((T, n), dtype=torch.float32, device=x_d.device)
    s = torch.empty_like(m)
    zy = torch.empty_like(m)
    for t in range(T):
        if stats_rows is not None and t in stats_rows:
            m[t], s[t], zy[t] = stats_rows[t]
            continue
        vp.vp_lmhead_ce_fwd(x_d, w_shards_d[t], tgt_d, starts[t], ends[t], m[t], s[t], zy[t])
    loss, lse, mean = vp.vp_ce_combine(m, s, zy, tgt_d, ignore_index)
    grads = {}
    for t in bwd_shards:
        grads[t] = vp.vp_lmhead_ce_bwd(x_d, w_shards_d[t], tgt_d, lse, starts[t], ends[t],
                                       grad_scale, ignore_index)
    torch.cuda.synchronize()
    return {"loss": loss, "lse": lse, "mean": mean, "m": m, "s": s, "zy": zy, "grads": grads}


def _rel_max_device(got_d, ref, rows_per_piece=2048):
    """max|got - ref| / max|ref| over whole tensors, with ``got_d`` (a GPU tensor) brought
    to the host a slab of rows at a time (a full-size gradient in fp64 would double host
    memory)."""
    num = den = 0.0
    finite = True
    for a in range(0, ref.shape[0], rows_per_piece):
        g = got_d[a:a + rows_per_piece].detach().cpu().numpy().astype(np.float64)
        r = ref[a:a + rows_per_piece]
        finite = finite and bool(np.isfinite(g).all())
        num = max(num, float(np.abs(g - r).max()))
        den = max(den, float(np.abs(r).max()))
    return (num / den if den > 0 else num), finite


def full_grads(out, t, x, w_shard, y, lse_ref, start, g):
    """Every element of shard t's dX partial and dW against the oracle (its dlogits formed
    token-chunked from the tokens' fp64 lse), with the bar's per-tensor denominator taken
    over the whole oracle tensor."""
    import time
    t0 = time.time()
    dx_ref, dw_ref = oracle.shard_grads_chunked(x, w_shard, y, lse_ref, start, g)
    log(f"  oracle dX/dW of shard {t} ({x.shape[0]} x {w_shard.shape[0]} x {x.shape[1]}): "
        f"{time.time() - t0:.1f} s")
    for name, got_d, ref in (("dX", out["grads"][t][0], dx_ref), ("dW", out["grads"][t][1], dw_ref)):
        e, finite = _rel_max_device(got_d, ref)
        log(f"  {name}_{t} (all {ref.shape[0]} x {ref.shape[1]}): max|d|/max|ref| {e:.3e} "
            f"(bar {GRAD_RTOL})")
        assert finite, f"{name}_{t}: non-finite values"
        assert e <= GRAD_RTOL, f"{name}_{t}: relative error {e} > {GRAD_RTOL}"


def embed_bwd_run(vp, ids, dout_bits, lo, hi, dw0):
    """vp_embed_bwd on the GPU, adding into a device copy of dw0."""
    dw = torch.from_numpy(np.ascontiguousarray(dw0, dtype=np.float32)).cuda()
    vp.vp_embed_bwd(dev_i64(ids), dev_bf16(dout_bits), lo, hi, dw)
    torch.cuda.synchronize()
    return dw


def embed_bwd_compare(got, base, want_sum, mag_sum, count, label):
    """got = base + the row sums, within the summation bound; rows with count 0 unchanged."""
    want = base.astype(np.float64) + want_sum
    bound = (count[:, None] + 1.0) * U * (np.abs(base).astype(np.float64) + mag_sum)
    err = np.abs(got - want)
    worst = float((err - bound).max())
    log(f"  {label}: {len(count)} rows, max abs err {err.max():.3e}, rel {rel_max(got, want):.3e}, "
        f"longest row {int(count.max()) if count.size else 0} tokens")
    assert worst <= 0.0, f"{label}: error above the summation bound by {worst:.3e}"
    assert rel_max(got, want) <= 1e-2
    untouched = count == 0
    assert np.array_equal(got[untouched], base[untouched].astype(np.float64)), \
        f"{label}: a row no owned id names was modified"


def embed_bwd_assert_rows(got, dw0, ids, dout, lo, rows, label):
    """Rows `rows` (local) of the result against dw0 + the oracle's row sums."""
    ids = np.asarray(ids, dtype=np.int64)
    count = np.array([(ids == lo + int(r)).sum() for r in rows], dtype=np.float64)
    embed_bwd_compare(got, dw0[rows], oracle.embed_shard_grad_rows(ids, dout, lo, rows),
                      oracle.embed_shard_grad_rows(ids, np.abs(dout), lo, rows), count, label)


def embed_bwd_full_check(vp, ids, dout_bits, lo, hi, dw0=None, label=""):
    """Every row of the shard against dw0 + the oracle's scatter-add."""
    n, h = dout_bits.shape
    ids = np.asarray(ids, dtype=np.int64)
    dw0 = np.zeros((hi - lo, h), np.float32) if dw0 is None else dw0
    got = host(embed_bwd_run(vp, ids, dout_bits, lo, hi, dw0))
    dout = vp_inputs.bf16_bits_to_f64(dout_bits)
    own = (ids >= lo) & (ids < hi)
    count = np.bincount(ids[own] - lo, minlength=hi - lo).astype(np.float64)
    embed_bwd_compare(got, dw0, oracle.embed_shard_grad(ids, dout, lo, hi),
                      oracle.embed_shard_grad(ids, np.abs(dout), lo, hi), count, label)
    return got
