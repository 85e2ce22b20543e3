"""Parity checking between the device pool and the CPU oracle's pool image.

Bar (applied per decode step):
  * packed bytes identical, except integer codes that differ by one step where
    the oracle's exact pre-rounding product Y*w lies within 1e-6 of a
    half-integer (a rounding tie); at most 1e-4 of the codes may be excused.
    An excused head is re-synchronised by writing the oracle's bytes into the
    device pool (data flows oracle -> device only);
  * readout o: relative L2 error <= 1e-4 against the oracle (per step, over
    all requests and heads) and per head <= 1e-3 of ||o|| + 0.02 ||m||, with
    m the readout magnitude sum_i |q_i| |S_ij| (compare_o).
"""
from __future__ import annotations

import dataclasses

import numpy as np

D = 128
TIE_WINDOW = 1e-6
MAX_EXCUSED_FRACTION = 1e-4
O_REL_L2 = 1e-4
O_WORST_HEAD = 1e-3
MAG_WEIGHT = 0.02


@dataclasses.dataclass
class StepReport:
    blocks_checked: int = 0
    blocks_mismatched: int = 0
    codes_checked: int = 0
    codes_excused: int = 0
    o_rel_l2: float = 0.0
    o_worst_head: float = 0.0
    detail: str = ""


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def compare_o(o_dev, o_ref, rep: StepReport, o_mag=None):
    """Readout bar.  Over the whole step: relative L2.  Per head: the error
    relative to ||o|| + MAG_WEIGHT ||m||, where m_j = sum_i |q_i| |S_ij| (the
    oracle's readout magnitude).  Both sides are sums of 128 products in
    different orders, so a head whose readout cancels (|o_j| << m_j) carries
    a rounding difference of order 2^-24 * 64 * m_j that ||o|| alone would
    not account for (|fl(x.y) - x.y| <= gamma_n |x|.|y|); with the weight
    below the per-head bound allows 2e-5 ||m|| on top of 1e-3 ||o||."""
    rep.o_rel_l2 = rel_l2(o_dev, o_ref)
    od = np.asarray(o_dev, np.float64).reshape(-1, D)
    orf = np.asarray(o_ref, np.float64).reshape(-1, D)
    den = np.linalg.norm(orf, axis=1)
    if o_mag is not None:
        den = den + MAG_WEIGHT * np.linalg.norm(np.asarray(o_mag, np.float64).reshape(-1, D), axis=1)
    num = np.linalg.norm(od - orf, axis=1)
    per = np.where(den > 0, num / np.maximum(den, 1e-300), num)
    rep.o_worst_head = float(per.max()) if per.size else 0.0


def _tie_analysis(orc, orc_pool, h, S, blk_ref, blk_dev):
    """Count differing codes of one block and how many of them sit on a tie.

    S: the oracle's updated fp32 state of this head before requantisation.
    Returns (n_codes_differing, n_excusable, other_bytes_differ).
    """
    kinds = orc_pool.head_kinds(h)
    unit, mode, sb = orc_pool.unit, orc_pool.scale_mode, orc_pool.scale_bits
    e_ref, r_ref, c_ref = orc.decode_block(kinds, unit, mode, blk_ref, scale_bits=sb)
    e_dev, r_dev, c_dev = orc.decode_block(kinds, unit, mode, blk_dev, scale_bits=sb)
    introw = np.array([kk <= 8 for kk in kinds])
    diff = e_ref != e_dev
    other = bool(np.any(diff[~introw])) or not np.array_equal(r_ref, r_dev) \
        or not np.array_equal(c_ref, c_dev)
    ndiff = int(np.count_nonzero(diff[introw]))
    if ndiff == 0:
        return 0, 0, other
    # the oracle's pre-rounding product Y*w in float64 (exact) for integer rows
    r = np.where(introw, r_ref, np.float32(1.0)).astype(np.float32)
    ir = (np.float32(1.0) / r).astype(np.float32)
    Y = (np.asarray(S, np.float32) * ir[:, None]).astype(np.float32)
    if mode == 0:
        mx = np.max(np.abs(np.where(introw[:, None], Y, np.float32(0))), axis=0).astype(np.float32)
        c0 = np.where(mx < np.finfo(np.float32).tiny, np.float32(1), mx).astype(np.float32)
        if sb == 16:   # the clip-free column factor is stored rounded up to bfloat16
            c0 = np.array([orc.bf16_up(float(x)) for x in c0], np.float32)
    else:
        c0 = np.ones(D, np.float32)
    e = (np.float32(1.0) / c0).astype(np.float32)
    qmax = np.array([(2 ** (int(kk) - 1) - 1) if kk <= 8 else 1 for kk in kinds], np.float32)
    w = (e[None, :] * qmax[:, None]).astype(np.float32)
    t = Y.astype(np.float64) * w.astype(np.float64)
    zr = e_ref.view(np.int32).astype(np.int64)
    zd = e_dev.view(np.int32).astype(np.int64)
    tie = np.abs(np.abs(t - np.floor(t)) - 0.5) < TIE_WINDOW
    ok = introw[:, None] & diff & tie & (np.abs(zr - zd) == 1)
    return ndiff, int(np.count_nonzero(ok)), other


def compare_pool(orc, orc_pool, dev_pool, slots, state_of, rep: StepReport, resync=True):
    """Compare every (slot, head) block of the listed slots, byte for byte.

    state_of(b, h) -> the oracle's fp32 state of request b, head h before
    requantisation (only called for blocks that differ).
    """
    H = orc_pool.num_heads
    bad_msgs = []
    for b, slot in enumerate(slots):
        slot = int(slot)
        if slot < 0:
            continue
        raw = dev_pool.qdr_read_raw(slot)
        base = slot * orc_pool.slot_stride
        ref = orc_pool.mem[base: base + orc_pool.slot_stride]
        rep.blocks_checked += H
        rep.codes_checked += H * D * D
        if np.array_equal(raw, ref):
            continue
        excused_here = 0
        for h in range(H):
            off, n = int(orc_pool.head_off[h]), orc_pool.block_size(h)
            bd, br = raw[off:off + n], ref[off:off + n]
            if np.array_equal(bd, br):
                continue
            rep.blocks_mismatched += 1
            ndiff, nex, other = _tie_analysis(orc, orc_pool, h, state_of(b, h), br, bd)
            if other or nex != ndiff or ndiff == 0:
                bad_msgs.append(f"slot {slot} head {h}: {ndiff} codes differ, {nex} at ties, "
                                f"other bytes differ: {other}")
            else:
                excused_here += nex
                raw[off:off + n] = br
        rep.codes_excused += excused_here
        if resync and excused_here:
            dev_pool.qdr_write_raw(slot, raw)
    if bad_msgs:
        rep.detail = "; ".join(bad_msgs[:8]) + (f" (+{len(bad_msgs) - 8} more)" if len(bad_msgs) > 8 else "")
    return rep


def step_state_fn(orc, orc_pool, prev_mem, slots, inputs):
    """state_of() for a decode step: re-run the oracle head step on the
    oracle's pre-step bytes to recover its un-requantised state."""
    q, k, v, beta, gate = inputs

    def state_of(b, h):
        slot = int(slots[b])
        off = slot * orc_pool.slot_stride + int(orc_pool.head_off[h])
        blk = prev_mem[off: off + orc_pool.block_size(h)]
        kinds = orc_pool.head_kinds(h)
        e0, r0, c0 = orc.decode_block(kinds, orc_pool.unit, orc_pool.scale_mode, blk,
                                      scale_bits=orc_pool.scale_bits)
        a = np.full(D, gate[b, h], np.float32) if gate.ndim == 2 else gate[b, h]
        _, _, _, _, S = orc.head_step(kinds, e0, r0, c0, orc_pool.omega[h], q[b, h], k[b, h],
                                      v[b, h], float(beta[b, h]), a,
                                      scale_mode=orc_pool.scale_mode, fit_iters=orc_pool.fit_iters,
                                      scale_bits=orc_pool.scale_bits)
        return S
    return state_of


def assert_step_ok(rep: StepReport, what: str):
    assert not rep.detail, f"{what}: {rep.detail}"
    assert rep.codes_excused <= MAX_EXCUSED_FRACTION * max(rep.codes_checked, 1), \
        f"{what}: {rep.codes_excused} excused codes of {rep.codes_checked}"
    assert rep.o_rel_l2 <= O_REL_L2, f"{what}: readout relative L2 {rep.o_rel_l2:.3e}"
    assert rep.o_worst_head <= O_WORST_HEAD, f"{what}: worst head readout relative L2 {rep.o_worst_head:.3e}"


def readout_row_sensitivity(orc, q, k, beta, a, eps=2.0 ** 12):
    """d o_t / d S_{t-1}[i, j] (the same for every column j), measured through
    the oracle's own decode step: an FP32-kind head whose stored state is
    eps * I takes one step with v = 0, and its readout divided by eps is the
    coefficient of each row (the step is linear in the stored state, and with
    v = 0 the stored state is its only input).  a: the gate as a per-row
    vector.  Returns float64 [128]."""
    d = len(q)
    S = (np.eye(d) * eps).astype(np.float32)
    kinds = np.full(d, 32, np.uint8)
    _, _, _, o, _ = orc.head_step(kinds, S.view(np.uint32), np.zeros(d, np.float32), np.ones(d, np.float32),
                                  np.ones(d, np.float32), q, k, np.zeros(d, np.float32), float(beta), a)
    return o.astype(np.float64) / eps
