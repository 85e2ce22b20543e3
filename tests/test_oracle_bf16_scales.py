"""Pins of the oracle's bfloat16 factor storage (16-bit r and c).

The rounding functions against a library routine (torch's float32 ->
bfloat16 conversion rounds to nearest even) and against their definition
(the smallest bfloat16 not below x); the requantiser against what the
rounding must guarantee (codes within +-q, stored factors bracketing the
fp32 ones, restore error within half a grid step); a state whose factors are
bfloat16 values already (identical codes in both widths); the block layout.
"""
import numpy as np
import pytest
import torch

D = 128


def bf16_of(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def test_nearest_matches_torch(orc):
    g = np.random.default_rng(1)
    x = np.concatenate([g.standard_normal(3000).astype(np.float32) * 10.0 ** g.integers(-20, 20, 3000),
                        # exact ties: a bfloat16 value plus half its last step
                        (np.float32(1.0) + np.float32(2.0 ** -8)) * np.float32([1, 3, 7, -5]),
                        np.float32([0.0, -0.0, 1e-30, 3.0e38])]).astype(np.float32)
    want = bf16_of(x)
    got = np.array([orc.bf16_nearest(float(v)) for v in x], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_up_is_smallest_bf16_not_below(orc):
    g = np.random.default_rng(2)
    x = np.abs(g.standard_normal(3000)).astype(np.float32) * np.float32(10.0) ** g.integers(-30, 30, 3000).astype(np.float32)
    x = np.concatenate([x, np.float32([1.0, 0.5, 2.0 ** -126, 1.0 + 2.0 ** -7])]).astype(np.float32)
    for v in x:
        u = orc.bf16_up(float(v))
        ub = np.float32(u).view(np.uint32)
        assert ub & 0xFFFF == 0                     # a bfloat16 value
        assert u >= v                               # not below x
        below = (ub - 0x10000).view(np.float32) if ub >= 0x10000 else np.float32(-1)
        assert below < v or u == v                  # the next bfloat16 down is below x


def _requant_both(orc, kinds, S, omega, mode, fit):
    e32, r32, c32, _ = orc.requant(kinds, S, omega, scale_mode=mode, fit_iters=fit)
    e16, r16, c16, _ = orc.requant(kinds, S, omega, scale_mode=mode, fit_iters=fit, scale_bits=16)
    return (e32, r32, c32), (e16, r16, c16)


@pytest.mark.parametrize("mode,fit", [(0, 0), (0, 1), (1, 0)])
def test_requant_guarantees(orc, mode, fit):
    from quantized_delta_rule_decode_amd import synth
    g = np.random.default_rng(3)
    kinds = g.choice(np.array([2, 4, 6, 8], np.uint8), size=D)
    S = synth.random_state(4, 1, 1)[0, 0]
    omega = g.lognormal(0, 1, D).astype(np.float32)
    (e32, r32, c32), (e16, r16, c16) = _requant_both(orc, kinds, S, omega, mode, fit)
    q = (2.0 ** (kinds.astype(np.int64) - 1) - 1)
    z = e16.view(np.int32).astype(np.int64)
    assert np.all(np.abs(z) <= q[:, None])
    for arr in (r16, c16):
        assert np.all(arr.view(np.uint32) & 0xFFFF == 0)
    assert np.all(r16 >= r32) and np.all(r16 <= r32 * (1 + 2.0 ** -7))
    ir = (np.float32(1) / r16).astype(np.float32)
    Y = (S * ir[:, None]).astype(np.float32)
    if mode == 0 and fit == 0:
        assert np.all(c16 >= np.abs(Y).max(axis=0))
    # restore: X = r c z / q, within half a grid step (plus rounding) of S
    if fit == 0:
        X = orc.dequant(kinds, e16, r16, c16, np.ones(D, np.float32)).astype(np.float64)
        step = (r16.astype(np.float64)[:, None] * c16.astype(np.float64)[None, :]) / q[:, None]
        assert np.all(np.abs(X - S) <= 0.5 * step * (1 + 1e-5) + 1e-30)


def test_representable_factors_give_identical_codes(orc):
    g = np.random.default_rng(5)
    kinds = g.choice(np.array([2, 4, 6, 8], np.uint8), size=D)
    S = np.where(g.random((D, D)) < 0.5, -1.0, 1.0).astype(np.float32)     # m_i = 1
    S[:, 7] *= np.float32(0.25)
    S[3] *= np.float32(4.0)
    m = np.abs(S).mean(axis=1)
    omega = (m / np.float32(4.0)).astype(np.float32)                        # r_i = 2 exactly
    (e32, r32, c32), (e16, r16, c16) = _requant_both(orc, kinds, S, omega, 0, 0)
    assert np.array_equal(r32, r16) and np.array_equal(c32, c16)
    assert np.array_equal(e32, e16)


def test_layout_and_roundtrip(orc):
    for b in (2, 4, 6, 8):
        k = np.full(D, b, np.uint8)
        assert orc.block_bytes(k, 0, 0, 16) == D * D * b // 8 + 512
        assert orc.block_bytes(k, 0, 1, 16) == D * D * b // 8 + 256
    assert orc.block_bytes(np.full(D, 16, np.uint8), 0, 0, 16) == 32768      # no factors
    g = np.random.default_rng(6)
    kinds = g.choice(np.array([2, 4, 6, 8, 16], np.uint8), size=D)
    from quantized_delta_rule_decode_amd import synth
    S = synth.random_state(7, 1, 1)[0, 0]
    for unit in (0, 1):
        kk = kinds if unit == 1 else np.full(D, 6, np.uint8)
        e, r, c, _ = orc.requant(kk, S, np.ones(D, np.float32), scale_bits=16)
        blob = orc.encode_block(kk, unit, 0, e, r, c, scale_bits=16)
        e2, r2, c2 = orc.decode_block(kk, unit, 0, blob, scale_bits=16)
        assert np.array_equal(e2, e) and np.array_equal(r2, r) and np.array_equal(c2, c)
