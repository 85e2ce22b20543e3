"""Host checks of the offline allocator: the lifetime weight against its
defining sum, the allocation against brute force (separable convex costs on
equally spaced candidates, where greedy marginal upgrades are optimal) and
against Lagrangian solutions, budget and pivot accounting."""
import itertools

import numpy as np
import pytest

from quantized_delta_rule_decode_amd import calib, synth


def test_lifetime_weight_is_the_geometric_sum():
    for ell in (0.0, -1e-6, -0.003, -0.05, -0.7, -5.0):
        J = 300
        direct = sum(np.exp(2 * j * ell) for j in range(J))
        assert calib.lifetime_weight(np.array([ell]), J)[0] == pytest.approx(direct, rel=1e-12)
    # ell -> -inf: only the j = 0 term survives; ell = 0: J terms of 1
    assert calib.lifetime_weight(np.array([-60.0]), 10)[0] == pytest.approx(1.0)
    assert calib.lifetime_weight(np.array([0.0]), 17)[0] == 17.0


def convex_costs(g, N, C):
    """Decreasing convex distortion curves on equally spaced widths."""
    steps = np.sort(g.uniform(0.01, 1.0, size=(N, C - 1)), axis=1)[:, ::-1]   # shrinking decrements
    base = g.uniform(1.0, 3.0, size=(N, 1))
    return np.concatenate([base, base - np.cumsum(steps, axis=1)], axis=1) + 3.0


def brute(L, D, bits, budget):
    N, C = D.shape
    best, arg = np.inf, None
    for ch in itertools.product(range(C), repeat=N):
        b = sum(bits[c] for c in ch)
        if b > budget:
            continue
        cost = sum(L[u] * D[u, c] for u, c in enumerate(ch))
        if cost < best - 1e-12:
            best, arg = cost, ch
    return best, arg


@pytest.mark.parametrize("seed", range(6))
def test_allocation_matches_brute_force_on_convex_costs(seed):
    g = np.random.default_rng(seed)
    bits = (4, 6, 8)
    N = 6
    L = g.uniform(0.5, 5.0, size=N)
    D = convex_costs(g, N, 3)
    for nominal in (4.0, 4.4, 5.0, 5.67, 6.0, 7.3, 8.0):
        kinds, piv = calib.allocate(L, D, bits, nominal, 0.0)
        assert not piv.any()
        ch = [bits.index(k) for k in kinds]
        cost = sum(L[u] * D[u, c] for u, c in enumerate(ch))
        best, _ = brute(L, D, bits, nominal * N)
        assert kinds.astype(int).sum() <= nominal * N
        assert cost == pytest.approx(best, rel=1e-12)


def test_allocation_reaches_lagrangian_solutions():
    g = np.random.default_rng(7)
    bits = np.array([2, 4, 6, 8])
    N = 200
    L = g.lognormal(0, 1.5, size=N)
    D = np.exp(-0.9 * bits[None, :] * g.uniform(0.5, 1.5, size=(N, 1))) * g.lognormal(0, 1, size=(N, 1))
    for lam in (1e-4, 1e-3, 1e-2, 1e-1):
        lag = np.argmin(L[:, None] * D + lam * bits[None, :], axis=1)
        budget_bits = bits[lag].sum()
        kinds, _ = calib.allocate(L, D, bits, budget_bits / N, 0.0)
        assert np.array_equal(kinds.astype(int), bits[lag])


def test_pivots_and_budget():
    g = np.random.default_rng(11)
    N = 500
    bits = (4, 6, 8)
    L = g.lognormal(0, 1, size=N)
    D = convex_costs(g, N, 3)
    kinds, piv = calib.allocate(L, D, bits, 6, 0.0139)
    n_piv = int(round(0.0139 * N))
    assert piv.sum() == n_piv and (kinds[piv] == synth.FP16).all()
    risk = L * D[:, -1]
    assert risk[piv].min() >= risk[~piv].max()                       # the riskiest units
    assert set(np.unique(kinds[~piv])) <= set(bits)
    assert kinds.astype(int).sum() <= 6 * N                          # pivots inside the budget
    assert kinds.astype(int).sum() > 6 * N - 4                       # and the budget is used
    with pytest.raises(ValueError):
        calib.allocate(L, D, bits, 4.05, 0.0139)                     # pivots + all-INT4 exceed it


@pytest.mark.parametrize("head", [True, False])
def test_row_impact_is_the_readout_sensitivity(orc, head):
    """The row-impact coefficient equals the sensitivity of the next readout
    to a row of the stored state, measured by perturbing the state through
    the oracle's decode step (not by evaluating a formula)."""
    import torch
    import parity
    g = np.random.default_rng(31 if head else 32)
    B, H, D = 3, 4, 128
    q = g.standard_normal((B, H, D))
    q /= np.linalg.norm(q, axis=-1, keepdims=True) * np.sqrt(D)
    k = g.standard_normal((B, H, D))
    k[..., :4] *= 8.0                                            # outlier key channels
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q[0, 0] = k[0, 0]                                            # a query along the key
    q, k = q.astype(np.float32), k.astype(np.float32)
    beta = g.uniform(0, 1, (B, H)).astype(np.float32)
    beta[1, 1] = 1.0
    gate = g.uniform(0.3, 1.0, (B, H) if head else (B, H, D)).astype(np.float32)
    coef = calib.row_impact(*(torch.from_numpy(x).double() for x in (q, k, beta, gate)), head).numpy()
    for b in range(B):
        for h in range(H):
            a = np.full(D, gate[b, h], np.float32) if head else gate[b, h]
            fd = parity.readout_row_sensitivity(orc, q[b, h], k[b, h], beta[b, h], a)
            scale = np.abs(a.astype(np.float64) * np.abs(q[b, h])).max() + np.abs(k[b, h]).max() * np.abs(q[b, h]).max()
            assert np.max(np.abs(coef[b, h] - fd)) <= 1e-5 * scale, (b, h, np.max(np.abs(coef[b, h] - fd)) / scale)
