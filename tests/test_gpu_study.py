"""The error-propagation study on the device path against the oracle.

A small study (24 heads, 2 sequences, 12 steps) runs through the C-ABI
(qdr_decode_step on a uniform INT6 row-absmax pool and an FP32 pool, qdr_unpack
after every step).  The test recomputes it with the oracle from the same
seeded inputs -- its own pools, its own error sums in float64, scipy's rank
correlation -- and compares the accumulated squared errors and rho.
"""
import numpy as np
import pytest
from scipy import stats

from quantized_delta_rule_decode_amd import qdr, study, synth

pytestmark = pytest.mark.gpu


def oracle_study(orc, sc):
    cfg = sc.synth_config()
    t = study.study_tables(sc)
    B, H = sc.B, sc.H
    p6 = orc.Pool(B, H, t["kinds"], np.ones((H, 128), np.float32), unit=orc.UNIT_HEAD,
                  gate=orc.GATE_SCALAR, scale_mode=orc.SCALE_ROW_ABSMAX).alloc()
    p32 = orc.Pool(B, H, np.full(H, 32, np.uint8), np.ones((H, 128), np.float32), unit=orc.UNIT_HEAD,
                   gate=orc.GATE_SCALAR, scale_mode=orc.SCALE_DUAL).alloc()
    slots = np.arange(B, dtype=np.int32)
    zero = np.zeros((B, H, 128, 128), np.float32)
    p6.pack(slots, zero)
    p32.pack(slots, zero)
    acc = np.zeros((B, H))
    for step in range(sc.T):
        ins = synth.step_inputs(cfg, t, step)
        _, bad6 = p6.step(slots, *ins, threads=8)
        _, bad32 = p32.step(slots, *ins, threads=8)
        assert bad6 == 0 and bad32 == 0
        d = p6.unpack(slots, threads=8).astype(np.float64) - p32.unpack(slots, threads=8).astype(np.float64)
        acc += (d * d).sum(axis=(2, 3))
    E = acc.sum(axis=0)
    hl = np.log(0.5) / np.log(t["alpha_head"].astype(np.float64))   # alpha^hl = 1/2
    return E, stats.spearmanr(hl, E).statistic


def test_study_matches_oracle(orc):
    import torch
    assert torch.cuda.is_available()
    qdr.load()
    sc = study.StudyConfig(H=24, B=2, T=12)
    assert sc.outliers
    print(f"study H={sc.H} B={sc.B} T={sc.T}", flush=True)
    r = study.run(sc)
    E_ref, rho_ref = oracle_study(orc, sc)
    assert (E_ref > 0).all()
    np.testing.assert_allclose(r["sq_error"], E_ref, rtol=1e-9, atol=0)
    assert r["rho"] == pytest.approx(rho_ref, abs=1e-12)
