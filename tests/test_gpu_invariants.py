"""The device step at the inputs where the pages fix its result.

Each case runs the HIP path through the C ABI at inputs where the delta rule
(Tutorial "STEPQuant：取代 KV cache 的状态，6-bit 量化精度不掉", §二) has a
known outcome, and checks that outcome on the device's own results, besides
the usual oracle parity of bytes and readout:

  * ||k|| = 1, beta = 1: the update writes v along k, k^T S_t = v^T, so with
    q = k the readout is v.  The device evaluates o = S'^T q + (q . beta k)
    delta, whose two terms cancel here; the bound below follows from the
    rounding of that form (u = 2^-24 per operation, 128-term fma chains);
  * beta = 0 with D = I: the state is unchanged -- exactly for FP32 and FP16
    heads and for the row-absmax integer codes, within half a grid step of
    the new factors under dual-axis factors (the row magnitude is recomputed
    from the restored state);
  * k = e_m: only row m changes and becomes v up to one rounding; every other
    row is the gated old row bit for bit; with q = e_m and beta = 1 the
    readout is that new row exactly;
  * diagonal gate entries a_i in {0, 1}: a row with a_i = 0 and k_i = 0 is
    erased, a row with a_i = 1 and k_i = 0 is kept bit for bit.
The FP32 kind stores S_t itself, so there the state checks read the updated
state back with qdr_unpack; the integer kinds are checked through the
readout and the oracle.
"""
import numpy as np
import pytest

from quantized_delta_rule_decode_amd import qdr, synth

import parity

pytestmark = pytest.mark.gpu
D = 128
U = 2.0 ** -24


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "device tests need a HIP GPU"
    qdr.load()
    return torch


def t_(torch, x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def unit(x):
    return (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)


# pools: (name, unit, kinds per head or per row, H)
def pool_kinds(name):
    g = np.random.default_rng(11)
    if name == "heads_int":
        return 0, np.array([2, 4, 6, 8], np.uint8), 4
    if name == "heads_float":
        return 0, np.array([16, 32, 6], np.uint8), 3
    if name == "heads_fp32":
        return 0, np.array([32, 32], np.uint8), 2
    k = g.choice(np.array([2, 4, 6, 8], np.uint8), size=(2, D), p=[0.3, 0.4, 0.2, 0.1])
    k[0, 5] = 16
    k[1, 70] = 32
    return 1, np.ascontiguousarray(k.reshape(-1)), 2


POOLS = ["heads_int", "heads_float", "heads_fp32", "rows_mixed"]
SCALES = [(0, 0), (0, 1), (1, 0)]


class Case:
    """A device pool and an oracle pool with the same packed start state."""

    def __init__(self, torch, orc, name, gate, scale, fit, n=3, seed=0):
        self.torch, self.orc = torch, orc
        self.unit, self.kinds, self.H = pool_kinds(name)
        g = np.random.default_rng(100 + seed)
        self.omega = g.lognormal(0, 1, (self.H, D)).astype(np.float32)
        kw = dict(unit=self.unit, gate=gate, scale_mode=scale, fit_iters=fit)
        self.dev = qdr.Pool(n, self.H, self.kinds, self.omega, **kw)
        self.ref = orc.Pool(n, self.H, self.kinds, self.omega, **kw).alloc()
        self.n, self.gate = n, gate
        rows16 = (self.kinds.reshape(self.H, D) == 16) if self.unit == 1 else \
            np.repeat((self.kinds == 16)[:, None], D, axis=1)
        S = synth.random_state(200 + seed, n, self.H)
        S = np.where(rows16[None, :, :, None], np.clip(S, -6e4, 6e4), S).astype(np.float32)
        self.slots = np.arange(n, dtype=np.int32)
        self.dev.qdr_pack(t_(torch, self.slots), t_(torch, S))
        self.ref.pack(self.slots, S)

    def head_kinds(self, h):
        return self.ref.head_kinds(h)

    def restored(self):
        """The device's current state, restored (qdr_unpack)."""
        out = self.torch.empty((self.n, self.H, D, D), dtype=self.torch.float32, device="cuda")
        self.dev.qdr_unpack(t_(self.torch, self.slots), out)
        return out.cpu().numpy()

    def step(self, q, k, v, beta, gate, what):
        """One step on both sides; oracle parity of bytes and readout."""
        prev = self.ref.mem.copy()
        ins = tuple(np.ascontiguousarray(x, np.float32) for x in (q, k, v, beta, gate))
        o = self.torch.full((self.n, self.H, D), 3.0, dtype=self.torch.float32, device="cuda")
        self.dev.qdr_decode_step(t_(self.torch, self.slots), *[t_(self.torch, x) for x in ins], o)
        o_ref, bad = self.ref.step(self.slots, *ins, threads=8)
        o_dev = o.cpu().numpy()
        rep = parity.StepReport()
        parity.compare_o(o_dev, o_ref, rep, self.ref.last_o_mag)
        parity.compare_pool(self.orc, self.ref, self.dev, self.slots,
                            parity.step_state_fn(self.orc, self.ref, prev, self.slots, ins), rep)
        parity.assert_step_ok(rep, what)
        assert bad == 0 and self.dev.qdr_poll_device_error() == 0
        return o_dev

    def gate_vec(self, gate):
        """The gate as a per-row vector for each (request, head)."""
        return np.broadcast_to(gate[..., None], (self.n, self.H, D)) if gate.ndim == 2 else gate


@pytest.mark.parametrize("name", POOLS)
@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("scale,fit", SCALES)
def test_unit_key_beta_one_reads_out_value(torch_dev, orc, name, gate, scale, fit):
    c = Case(torch_dev, orc, name, gate, scale, fit, seed=1)
    g = np.random.default_rng(21)
    n, H = c.n, c.H
    k = unit(g.standard_normal((n, H, D)))
    v = (g.standard_normal((n, H, D)) * g.lognormal(0, 1, (1, H, D))).astype(np.float32)
    beta = np.ones((n, H), np.float32)
    gate_in = g.uniform(0.5, 1.0, (n, H, D) if gate else (n, H)).astype(np.float32)
    X = c.restored()
    Sp = (c.gate_vec(gate_in)[..., None].astype(np.float32) * X).astype(np.float32)   # D S_{t-1}
    o = c.step(k, k, v, beta, gate_in, f"I1 {name} gate={gate} scale={scale} fit={fit}")
    # |o - v| <= 2^-16 (2 sum_i |k_i S'_ij| + |v_j|): the two 128-term chains
    # (u and S'^T q), delta = v - u, q . beta k = 1 + O(128 u), each within
    # 256 u of its magnitude
    A = np.einsum("bhi,bhij->bhj", np.abs(k.astype(np.float64)), np.abs(Sp.astype(np.float64)))
    bound = 256 * U * (2 * A + np.abs(v))
    err = np.abs(o.astype(np.float64) - v)
    assert np.all(err <= bound), f"worst |o - v| / bound = {np.max(err / bound):.3f}"
    # the FP32 heads store S_t itself: k^T S_t = v^T within the same kind of bound
    S1 = c.restored()
    for h in range(H):
        if not np.all(c.head_kinds(h) == 32):
            continue
        kS = np.einsum("bi,bij->bj", k[:, h].astype(np.float64), S1[:, h].astype(np.float64))
        A1 = np.einsum("bi,bij->bj", np.abs(k[:, h].astype(np.float64)), np.abs(S1[:, h].astype(np.float64)))
        assert np.all(np.abs(kS - v[:, h]) <= 256 * U * (2 * A + np.abs(v))[:, h] + 256 * U * A1)


@pytest.mark.parametrize("name", POOLS)
@pytest.mark.parametrize("scale,fit", SCALES)
def test_identity_gate_zero_beta_keeps_state(torch_dev, orc, name, scale, fit):
    c = Case(torch_dev, orc, name, 0, scale, fit, seed=2)
    g = np.random.default_rng(22)
    n, H = c.n, c.H
    before = [c.dev.qdr_read_raw(s) for s in c.slots]
    X0 = c.restored()
    for step in range(3):
        q = (unit(g.standard_normal((n, H, D))) / np.sqrt(D)).astype(np.float32)
        k = unit(g.standard_normal((n, H, D)))
        v = g.standard_normal((n, H, D)).astype(np.float32)
        X_prev = c.restored()
        c.step(q, k, v, np.zeros((n, H), np.float32), np.ones((n, H), np.float32),
               f"beta=0 D=I {name} scale={scale} fit={fit} step {step}")
        X = c.restored()
        for s in c.slots:
            raw = c.dev.qdr_read_raw(s)
            for h in range(H):
                kinds = c.head_kinds(h)
                fl = kinds > 8
                if fl.all():
                    # FP32 / FP16 heads: bytes unchanged
                    assert np.array_equal(c.dev.block(raw, h), c.dev.block(before[s], h))
                elif fl.any():
                    # float rows of a row-unit head keep their values
                    assert np.array_equal(X[s, h][fl].view(np.uint32), X0[s, h][fl].view(np.uint32))
                if scale == 1:
                    # row-absmax integer codes are kept
                    e0, _, _ = orc.decode_block(kinds, c.unit, scale, c.dev.block(before[s], h))
                    e1, _, _ = orc.decode_block(kinds, c.unit, scale, c.dev.block(raw, h))
                    assert np.array_equal(e0[~fl], e1[~fl])
                elif fit == 0 and not fl.all():
                    # dual-axis: within half a grid step of the new factors
                    _, r1, c1 = orc.decode_block(kinds, c.unit, scale, c.dev.block(raw, h))
                    qm = np.where(fl, 1, 2.0 ** (kinds.astype(np.int64) - 1) - 1)
                    half = 0.5 * r1.astype(np.float64)[:, None] * c1.astype(np.float64)[None, :] / qm[:, None]
                    d = np.abs(X[s, h].astype(np.float64) - X_prev[s, h].astype(np.float64))
                    assert np.all(d[~fl] <= (half * (1 + 1e-5))[~fl])


@pytest.mark.parametrize("name", POOLS)
@pytest.mark.parametrize("gate", [0, 1])
@pytest.mark.parametrize("scale,fit", SCALES)
def test_basis_key_rewrites_one_row(torch_dev, orc, name, gate, scale, fit):
    c = Case(torch_dev, orc, name, gate, scale, fit, seed=3)
    g = np.random.default_rng(23)
    n, H = c.n, c.H
    m = np.array([[[5, 64, 127, 0][(b + h) % 4] for h in range(H)] for b in range(n)])
    e_m = np.zeros((n, H, D), np.float32)
    for b in range(n):
        for h in range(H):
            e_m[b, h, m[b, h]] = 1.0
    v = g.standard_normal((n, H, D)).astype(np.float32)
    gate_in = g.uniform(0.3, 1.0, (n, H, D) if gate else (n, H)).astype(np.float32)
    X = c.restored()
    Sp = (c.gate_vec(gate_in)[..., None].astype(np.float32) * X).astype(np.float32)
    o = c.step(e_m, e_m, v, np.ones((n, H), np.float32), gate_in,
               f"k=e_m {name} gate={gate} scale={scale} fit={fit}")
    S1 = c.restored()
    for b in range(n):
        for h in range(H):
            mm = m[b, h]
            # the readout is the new row m: v up to one rounding of delta and one of the add
            assert np.all(np.abs(o[b, h] - v[b, h]) <= 2 * U * (np.abs(v[b, h]) + 2 * np.abs(Sp[b, h, mm])))
            if np.all(c.head_kinds(h) == 32):
                others = np.arange(D) != mm
                assert np.array_equal(S1[b, h][others].view(np.uint32), Sp[b, h][others].view(np.uint32))
                assert np.array_equal(o[b, h].view(np.uint32), S1[b, h, mm].view(np.uint32))


@pytest.mark.parametrize("name", POOLS)
@pytest.mark.parametrize("scale,fit", SCALES)
def test_binary_diagonal_gate(torch_dev, orc, name, scale, fit):
    c = Case(torch_dev, orc, name, 1, scale, fit, seed=4)
    g = np.random.default_rng(24)
    n, H = c.n, c.H
    a = (g.random((n, H, D)) < 0.5).astype(np.float32)
    a[..., :4] = 0.0
    a[..., 4:8] = 1.0
    kz = g.random((n, H, D)) < 0.4                 # rows the key does not touch
    kz[..., :8] = True
    k = g.standard_normal((n, H, D))
    k[kz] = 0.0
    k = unit(k)
    q = (unit(g.standard_normal((n, H, D))) / np.sqrt(D)).astype(np.float32)
    v = g.standard_normal((n, H, D)).astype(np.float32)
    X = c.restored()
    c.step(q, k, v, g.uniform(0, 1, (n, H)).astype(np.float32), a, f"a in {{0,1}} {name} scale={scale} fit={fit}")
    S1 = c.restored()
    for b in range(n):
        for h in range(H):
            if not np.all(c.head_kinds(h) == 32):
                continue
            erased = (a[b, h] == 0) & kz[b, h]
            kept = (a[b, h] == 1) & kz[b, h]
            assert np.all(S1[b, h][erased] == 0.0)
            assert np.array_equal(S1[b, h][kept].view(np.uint32), X[b, h][kept].view(np.uint32))
