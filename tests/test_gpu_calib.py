"""Offline calibration on the device path against the oracle.

calib.calibrate runs the FP32 trajectories, the omega and lifetime statistics
and the distortion of every candidate width through the C-ABI.  The test
recomputes every statistic with the oracle's pools from the same seeded
inputs (its own float64 sums, the lifetime weight as the explicit sum, the
row impact omega as the measured sensitivity of the next readout to each row
of the stored state, through the oracle's step) and checks the allocation the
package derives from them.
"""
import numpy as np
import pytest

from quantized_delta_rule_decode_amd import calib, qdr, synth

import parity

pytestmark = pytest.mark.gpu


def oracle_calib(orc, cc):
    cfg = cc.synth_config()
    t = synth.static_tables(cfg)
    B, H = cc.n_seq, cc.H
    head = cc.unit == synth.UNIT_HEAD
    slots = np.arange(B, dtype=np.int32)
    f32 = orc.Pool(B, H, np.full(H, 32, np.uint8), np.ones((H, 128), np.float32), unit=orc.UNIT_HEAD,
                   gate=cfg.gate, scale_mode=orc.SCALE_DUAL).alloc()
    f32.pack(slots, np.zeros((B, H, 128, 128), np.float32))
    sample_at = sorted({max(1, int(round(f * cc.T))) for f in cc.samples})
    samples, logs, coefs = [], [], []
    for step in range(cc.T):
        q, k, v, beta, gate = synth.step_inputs(cfg, t, step)
        logs.append(np.log(gate.astype(np.float64)))
        if step > 0:
            # the readout's sensitivity to each row of the stored state,
            # measured through the oracle's step (a perturbed stored state)
            c = np.empty((B, H, 128))
            for b in range(B):
                for h in range(H):
                    a = np.full(128, gate[b, h], np.float32) if head else gate[b, h]
                    c[b, h] = parity.readout_row_sensitivity(orc, q[b, h], k[b, h], beta[b, h], a)
            coefs.append(c * c)
        _, bad = f32.step(slots, q, k, v, beta, gate, threads=8)
        assert bad == 0
        if step + 1 in sample_at:
            samples.append(f32.unpack(slots, threads=8))
    ell = np.mean(logs, axis=(0, 1)).reshape(-1)
    om = np.mean(np.concatenate(coefs, axis=0), axis=0)
    om = np.maximum(om / om.mean(axis=1, keepdims=True), 1e-3).astype(np.float32)
    L = np.array([sum(np.exp(2.0 * j * e) for j in range(cc.horizon)) for e in ell])
    cands = calib.CANDIDATES[cc.nominal]
    n_units = H if head else H * 128
    D = np.zeros((n_units, len(cands)))
    for ci, b in enumerate(cands):
        p = orc.Pool(B, H, np.full(n_units, b, np.uint8), om, unit=cc.unit, gate=cfg.gate,
                     scale_mode=orc.SCALE_DUAL).alloc()
        rows = np.zeros((H, 128))
        for S in samples:
            p.pack(slots, S, threads=8)
            d = p.unpack(slots, threads=8).astype(np.float64) - S.astype(np.float64)
            rows += (d * d).sum(axis=(0, 3))
        rows /= B * len(samples)
        if head:
            D[:, ci] = (rows * om.astype(np.float64)).sum(axis=1) / 128 ** 2
        else:
            D[:, ci] = (rows / 128).reshape(-1)
    return ell, om, L, D


@pytest.mark.parametrize("unit", ["head", "row"])
def test_calibration_matches_oracle(orc, unit):
    import torch
    assert torch.cuda.is_available()
    qdr.load()
    if unit == "head":
        cc = calib.CalibConfig(unit=synth.UNIT_HEAD, H=10, n_seq=2, T=16, nominal=6, pivot_frac=0.1, horizon=256)
    else:
        cc = calib.CalibConfig(unit=synth.UNIT_ROW, H=2, n_seq=2, T=16, nominal=4, pivot_frac=0.01, horizon=256)
    print(f"calibration unit={unit} H={cc.H} n_seq={cc.n_seq} T={cc.T}", flush=True)
    r = calib.calibrate(cc)
    ell, om, L, D = oracle_calib(orc, cc)
    np.testing.assert_allclose(r["ell"], ell, rtol=1e-12, atol=0)
    np.testing.assert_allclose(r["L"], L, rtol=1e-9, atol=0)
    np.testing.assert_allclose(r["omega"], om, rtol=1e-5, atol=0)
    np.testing.assert_allclose(r["D"], D, rtol=1e-3, atol=0)
    kinds, piv = calib.allocate(L, D, calib.CANDIDATES[cc.nominal], cc.nominal, cc.pivot_frac)
    assert np.array_equal(r["kinds"], kinds) and np.array_equal(r["pivot"], piv)
    assert (D[:, :-1] >= D[:, 1:]).all()          # wider codes, less distortion
