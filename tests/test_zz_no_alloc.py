"""The allocation-free forward (vp_lmhead_ce_fwd_noalloc) against the workspace form.

vp_lmhead_ce_fwd_noalloc runs the same kernels as vp_lmhead_ce_fwd with the workspace
taken from the library's fixed per-GPU scratch buffer.  Two calls in a row (the second on
a smaller, ragged problem, so it runs over what the first left in the buffer) must give
the workspace form's statistics bit for bit, and those are checked against the oracle
too; a problem whose workspace exceeds the buffer is refused before anything launches.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import vp_inputs
from gpu_util import assert_stats_close, dev_bf16, dev_i64, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vp():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vocab_lm_head_amd
    return vocab_lm_head_amd


def _case(vp, n, h, V, lo, hi, seed):
    """Both forms on the same seeded inputs; returns (noalloc outputs, workspace outputs,
    the host inputs)."""
    import torch
    r = np.random.default_rng(seed)
    x_bits = vp_inputs.f32_to_bf16_bits(r.standard_normal((n, h)).astype(np.float32))
    w_bits = vp_inputs.f32_to_bf16_bits(
        (r.standard_normal((hi - lo, h)) * (3.0 / np.sqrt(h))).astype(np.float32))
    y = r.integers(0, V, n).astype(np.int64)
    y[: min(n, 4)] = [lo, hi - 1, lo + (hi - lo) // 2, -100][: min(n, 4)]
    x, w, yd = dev_bf16(x_bits), dev_bf16(w_bits), dev_i64(y)
    outs = [tuple(torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(3))
            for _ in range(2)]
    vp.vp_lmhead_ce_fwd_noalloc(x, w, yd, lo, hi, *outs[0])
    vp.vp_lmhead_ce_fwd(x, w, yd, lo, hi, *outs[1])
    torch.cuda.synchronize()
    return outs, (x_bits, w_bits, y)


def test_noalloc_matches_workspace_form_twice(vp):
    import torch
    ws1 = vp.vp_lmhead_ce_fwd_workspace(8192, 1024, 16032, 2 * 16032)
    ws2 = vp.vp_lmhead_ce_fwd_workspace(1000, 256, 1500, 3000)
    assert ws2 < ws1 <= vp.NOALLOC_SCRATCH_BYTES
    log(f"  workspace bytes: first call {ws1}, second call {ws2}, "
        f"scratch {vp.NOALLOC_SCRATCH_BYTES}")
    for k, (n, h, V, lo, hi) in enumerate([(8192, 1024, 8 * 16032, 16032, 2 * 16032),
                                           (1000, 256, 4500, 1500, 3000)]):
        (na, ws), (x_bits, w_bits, y) = _case(vp, n, h, V, lo, hi, seed=40 + k)
        for name, u, v in zip(("m", "s", "zy"), na, ws):
            assert torch.equal(u, v), f"call {k}: {name} differs from the workspace form"
        x = vp_inputs.bf16_bits_to_f64(x_bits)
        w = vp_inputs.bf16_bits_to_f64(w_bits)
        ref = oracle.shard_stats(oracle.logits(x, w), y, lo)
        assert_stats_close(tuple(host(t) for t in na), ref, f"call {k} ({n} x {hi - lo} x {h})")
        log(f"  call {k}: bit-identical to vp_lmhead_ce_fwd")


def test_noalloc_refuses_more_than_its_scratch(vp):
    import torch
    n, h, lo, hi = 4096, 8, 0, 256000   # 2000 slices x 4096 tokens x 12 B > 64 MiB
    assert vp.vp_lmhead_ce_fwd_workspace(n, h, lo, hi) > vp.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((n, h), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((hi - lo, h), dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(n, dtype=torch.int64, device="cuda")
    outs = tuple(torch.full((n,), 7.0, device="cuda") for _ in range(3))
    with pytest.raises(vp.VPError) as e:
        vp.vp_lmhead_ce_fwd_noalloc(x, w, y, lo, hi, *outs)
    assert e.value.status == vp.VP_ERR_SCRATCH
    torch.cuda.synchronize()
    assert all(bool((t == 7.0).all()) for t in outs), "a refused call touched an output"
