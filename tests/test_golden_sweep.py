"""The scaling sweep's stored oracle values still match the generators and the oracle
(the smallest shape recomputed on the CPU): a change to ``vp_inputs.sweep_inputs`` or to
the sampled rows without regenerating ``tests/golden/oracle_sweep.npz`` fails here."""
import os

import numpy as np

import oracle
import vp_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_sweep.npz")


def test_sweep_golden_covers_every_shape():
    gold = np.load(GOLDEN)
    for N, H in vp_inputs.SWEEP_SHAPES:
        assert gold[f"{N}x{H}_loss"].shape == (N,)
        assert gold[f"{N}x{H}_dx"].shape == (4, H)
        assert gold[f"{N}x{H}_dw"].shape[1] == H


def test_sweep_golden_smallest_shape_recomputed():
    N, H, Vs, T = 1024, 4096, 16032, 8
    gold = np.load(GOLDEN)
    xb, wb, y = vp_inputs.sweep_inputs(N, H, Vs, T)
    x, w = vp_inputs.bf16_bits_to_f64(xb), vp_inputs.bf16_bits_to_f64(wb)
    m0, s0, zy0 = oracle.shard_stats(oracle.logits(x, w), y, 0)
    ones = np.ones(N)
    loss, lse, _ = oracle.combine_triples(
        np.stack([m0] + [ones] * (T - 1)), np.stack([s0] + [1000.0 * ones] * (T - 1)),
        np.stack([zy0] + [0.0 * ones] * (T - 1)), y)
    assert np.allclose(gold[f"{N}x{H}_loss"], loss, rtol=0, atol=1e-9)
    rows, cols = vp_inputs.sweep_samples(N, H, y, Vs)
    dw = oracle.dz_cols(x, w[cols], cols, y, lse, 1.0 / N).T @ x
    assert np.allclose(gold[f"{N}x{H}_dw"], dw, rtol=1e-6, atol=1e-9)
