"""The gradient GEMMs' four launch forms, each at a shape that takes it, through the whole
CE path of one shard (T = 1, every token's loss and both gradients in full) against the
oracle:

  128 x 128 tiles, both products in one launch: the small LM (N 4096, H 512, Vs 3200)
      and a ragged N 300, H 136, Vs 700;
  256 x 256 tiles, both split over K in one grouped launch: N 2048, H 512, Vs 9000;
  only dX split over K: N 256, H 512, Vs 16000;
  only dW split over K: N 12000, H 64, Vs 900.

The workspace the library asks for names the form that runs (the fp32 partials of the
split products, none for the others); each case checks it first, with the sizes worked
out by hand in the boundary test.  The comparator's backward (stored logits) shares these
launches; the small-LM case runs it too.  Same bars as the other parity tests."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import vp_inputs
from gpu_util import (assert_grad_close, assert_loss_close, dev_bf16, dev_i64, host, log,
                      run_ce_path)

pytestmark = pytest.mark.gpu


def _r256(b):
    return -(-b // 256) * 256


def _r64(e):
    return -(-e // 64) * 64


def _bufs(n, h, vs):
    return (_r256(h * _r64(n) * 2) + _r256(h * _r64(vs) * 2) + _r256(n * _r64(vs) * 2)
            + _r256(vs * _r64(n) * 2))


CASES = [
    ("small_tiles_small_lm", 4096, 512, 3200, 0),
    ("small_tiles_ragged", 300, 136, 700, 0),
    ("grouped_split", 2048, 512, 9000, _r256(7 * 2048 * 512 * 4) + _r256(2 * 9000 * 512 * 4)),
    ("dx_split", 256, 512, 16000, _r256(16 * 256 * 512 * 4)),
    ("dw_split", 12000, 64, 900, _r256(16 * 900 * 64 * 4)),
]


@pytest.fixture(scope="module")
def vp():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_lm_head_amd
    return vocab_lm_head_amd


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gradient_launch_form(vp, case):
    name, N, H, Vs, partials = case
    assert vp.vp_lmhead_ce_bwd_workspace(N, H, 0, Vs) == _bufs(N, H, Vs) + partials, name
    r = np.random.default_rng(N + H + Vs)
    xb = vp_inputs.f32_to_bf16_bits(r.standard_normal((N, H)).astype(np.float32))
    wb = vp_inputs.f32_to_bf16_bits(
        r.standard_normal((Vs, H)).astype(np.float32) * np.float32(3.0 / math.sqrt(H)))
    y = r.integers(0, Vs, N).astype(np.int64)
    y[r.random(N) < 0.1] = oracle.DEFAULT_IGNORE_INDEX
    log(f"  {name}: N={N} H={H} Vs={Vs}")
    x, w = vp_inputs.bf16_bits_to_f64(xb), vp_inputs.bf16_bits_to_f64(wb)
    z = oracle.logits(x, w)
    loss, lse, _ = oracle.dense_ce(z, y)
    dz = oracle.dense_dlogits(z, y)
    dx_ref, dw_ref = oracle.shard_grads(x, w, dz)
    x_d, w_d, y_d = dev_bf16(xb), dev_bf16(wb), dev_i64(y)
    g = oracle.mean_scale(y)
    out = run_ce_path(vp, x_d, [w_d], [0], [Vs], y_d, g, bwd_shards=[0])
    assert_loss_close(host(out["loss"]), loss)
    assert_grad_close(host(out["grads"][0][0]), dx_ref, f"dX ({name})")
    assert_grad_close(host(out["grads"][0][1]), dw_ref, f"dW ({name})")
    if name == "small_tiles_small_lm":
        # the stored-logits backward goes through the same gradient launch
        import torch
        logits = vp.vp_lmhead_logits(x_d, w_d, 0, Vs)
        dx_c, dw_c = vp.vp_logits_ce_bwd(logits, x_d, w_d, y_d, out["lse"], 0, Vs, g)
        torch.cuda.synchronize()
        assert_grad_close(host(dx_c), dx_ref, "dX (stored logits)")
        assert_grad_close(host(dw_c), dw_ref, "dW (stored logits)")
