"""The C ABI used from C++ alone (tests/c_abi/vp_step.cpp: hipMalloc'd buffers, a stream of
its own, no torch): every shard's forward, the combine and every shard's backward, against
the oracle on the same bf16 inputs.  Same bars as the other parity tests.

The program is built with the library (``vocab_lm_head_amd/build.py``); this test only runs
it, in a child process."""
from __future__ import annotations

import math
import os
import subprocess

import numpy as np
import pytest

import oracle
import vp_inputs
from gpu_util import assert_grad_close, assert_loss_close, log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROGRAM = os.path.join(ROOT, "tests", "c_abi", "vp_step")


@pytest.fixture(scope="module")
def program():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(PROGRAM):
        pytest.fail(f"{PROGRAM} is not built (python vocab_lm_head_amd/build.py)")
    return PROGRAM


@pytest.mark.parametrize("N,H,V,T", [(300, 136, 2100, 3), (4096, 512, 6400, 2)])
def test_step_through_the_c_abi(program, tmp_path, N, H, V, T):
    """Ragged tiles (300 x 136, three shards of 700) and the small-LM shape, whose gradient
    GEMMs run as 128 x 128 tiles in one launch; 10% of the targets ignored."""
    r = np.random.default_rng(N + V)
    xb = vp_inputs.f32_to_bf16_bits(r.standard_normal((N, H)).astype(np.float32))
    wb = vp_inputs.f32_to_bf16_bits(
        r.standard_normal((V, H)).astype(np.float32) * np.float32(3.0 / math.sqrt(H)))
    y = r.integers(0, V, N).astype(np.int64)
    y[r.random(N) < 0.1] = oracle.DEFAULT_IGNORE_INDEX
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        np.array([N, H, V, T, oracle.DEFAULT_IGNORE_INDEX], dtype=np.int64).tofile(f)
        xb.tofile(f)
        wb.tofile(f)
        y.tofile(f)
    log(f"  C-ABI program: N={N} H={H} V={V} T={T}")
    p = subprocess.run([program, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, f"vp_step failed ({p.returncode}): {p.stderr}"
    out = np.fromfile(dst, dtype=np.float32).astype(np.float64)
    assert out.size == 2 * N + 1 + T * N * H + V * H
    loss_g, lse_g, mean_g = out[:N], out[N:2 * N], out[2 * N]
    dx_g = out[2 * N + 1:2 * N + 1 + T * N * H].reshape(T, N, H)
    dw_g = out[2 * N + 1 + T * N * H:].reshape(V, H)

    x, w = vp_inputs.bf16_bits_to_f64(xb), vp_inputs.bf16_bits_to_f64(wb)
    z = oracle.logits(x, w)
    loss, lse, mean = oracle.dense_ce(z, y)
    dz = oracle.dense_dlogits(z, y)
    assert_loss_close(loss_g, loss)
    assert_loss_close(lse_g, lse, "lse")
    assert abs(mean_g - mean) <= 2e-3
    for t in range(T):
        a, b = oracle.shard_range(V, T, t)
        dxr, dwr = oracle.shard_grads(x, w[a:b], dz[:, a:b])
        assert_grad_close(dx_g[t], dxr, f"dX partial {t}")
        assert_grad_close(dw_g[a:b], dwr, f"dW {t}")
