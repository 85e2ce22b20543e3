"""Offline calibration and lifetime-aware bit allocation.

Produces the static tables the decode step consumes -- the storage kind of
every unit (heads for GDN, key rows of every head for KDA) and the row-impact
scores omega -- from calibration trajectories, following the offline stage
of the pages (Tutorial §三 lifetime weight and row impact, §四 allocation and
pivots; Review (ai-trend), Method; Review (singularity-lens), calibration
paragraphs).  Synthetic sequences of the seeded generators stand in for the
pages' 32 WikiText-2 segments of 2,048 tokens (no model or dataset here).

Steps, on the device path (decode steps, pack and unpack through the C-ABI):
  1. run the unquantised delta rule (FP32-kind pool) over n_seq sequences of
     T steps from zero, keeping the states at the sample steps;
  2. mean log-retention of each unit, ell_u = mean over sequences and steps of
     log alpha (GDN: the head's scalar gate) or log a_i (KDA: the row's
     diagonal gate entry);
  3. lifetime weight L_u = sum_{j=0}^{J-1} exp(2 j ell_u) over a finite
     horizon of J steps (the geometric series of the squared retention: how
     much of an error injected now is still in the state j steps later);
  4. row impact omega_{h,i}: a perturbation of row i of the stored state
     reaches the next readout through that step's transform,
     o_t = (A_t S_{t-1} + ...)^T q_t with A_t = (I - beta k k^T) D_t, so its
     coefficient is (A_t^T q_t)_i = d_i (q_i - beta k_i (k . q)); omega is its
     square averaged over the calibration steps, normalised to mean 1 per head
     and floored at 1e-3 (the row factor divides by it);
  5. distortion D_u(b) of every candidate width b: the sampled states are
     packed into a pool whose every unit has kind b (dual-axis scales with the
     omega of step 4) and unpacked; GDN heads take the row-sensitivity-
     weighted mean squared error (1/128^2) sum_i omegã_i sum_j (S^ - S)^2,
     KDA rows the row's mean squared error (1/128) sum_j (S^ - S)^2, averaged
     over samples;
  6. allocation (allocate()): the riskiest units -- largest L_u * D_u at the
     widest integer candidate -- become FP16 pivots; the others get
     candidate widths minimising sum_u L_u D_u(b_u) under the average-bit
     budget (pivots counted at 16 bits), by greedy upgrades along each
     unit's lower convex hull of (bits, L_u D_u).
Candidates: {2,4,6,8} for a nominal 4-bit budget, {4,6,8} for 6-bit.

Run: python -m quantized_delta_rule_decode_amd.calib [--unit head|row ...]
writes the tables (.npz) and prints one JSON line that also compares the
allocation with a uniform one of the same budget on held-out sequences.
"""
from __future__ import annotations

import argparse
import dataclasses
import heapq
import json
import sys
import time

import numpy as np

from . import qdr, synth

CANDIDATES = {4: (2, 4, 6, 8), 6: (4, 6, 8)}
PIVOT_BITS = 16


@dataclasses.dataclass(frozen=True)
class CalibConfig:
    unit: int = synth.UNIT_HEAD      # UNIT_HEAD: GDN heads, scalar gate; UNIT_ROW: KDA rows, diagonal gate
    H: int = 2304
    n_seq: int = 8
    T: int = 256
    nominal: int = 6
    pivot_frac: float = 0.0139       # share of units kept in FP16 (1.39% of the GDN model's heads)
    horizon: int = 2048              # J of the lifetime weight (the calibration segment length)
    samples: tuple = (0.5, 1.0)      # state samples at these fractions of T
    outliers: bool = True
    fit_iters: int = 0               # column-factor refits of every quantised pool (0: clip-free c = max |Y|)
    seed_id: int = 11

    def synth_config(self, held_out: bool = False) -> synth.Config:
        head = self.unit == synth.UNIT_HEAD
        sid = self.seed_id + (100 if held_out else 0)
        return synth.Config(sid, f"calib_{'gdn' if head else 'kda'}_h{self.H}", self.n_seq, self.H, self.n_seq,
                            self.unit, synth.GATE_SCALAR if head else synth.GATE_DIAG, synth.SCALE_DUAL,
                            self.T, 0, self.outliers, "per_head" if head else "per_row",
                            device_inputs=self.n_seq * self.H > 4096)

    @property
    def n_units(self) -> int:
        return self.H if self.unit == synth.UNIT_HEAD else self.H * qdr.DIM


def lifetime_weight(ell, horizon: int) -> np.ndarray:
    """L = sum_{j=0}^{J-1} exp(2 j ell) (J = horizon) in closed form; ell <= 0."""
    x = 2.0 * np.asarray(ell, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        L = np.expm1(horizon * x) / np.expm1(x)
    return np.where(x == 0.0, float(horizon), L)


def _hull(bits, cost):
    """Indices of the lower convex hull of the points (bits[k], cost[k]),
    bits increasing, keeping only points that lower the cost."""
    idx = [0]
    for k in range(1, len(bits)):
        if cost[k] >= cost[idx[-1]]:
            continue
        while len(idx) >= 2:
            a, b = idx[-2], idx[-1]
            # b is above the segment a -> k: drop it
            if (cost[b] - cost[a]) * (bits[k] - bits[a]) >= (cost[k] - cost[a]) * (bits[b] - bits[a]):
                idx.pop()
            else:
                break
        idx.append(k)
    return idx


def allocate(L, D, cand_bits, nominal, pivot_frac):
    """Kinds of N units from lifetime weights L [N] and distortions D [N, C]
    (column c: candidate width cand_bits[c], increasing).

    Returns (kinds uint8 [N], pivot mask [N]).  Pivots: the round(pivot_frac N)
    units of largest L * D[:, -1] (ties: lower index first), stored as FP16.
    Budget: mean code bits over all units <= nominal, pivots at 16 bits.
    The rest start at the narrowest candidate and take the upgrade with the
    largest cost decrease per bit, along their convex hulls, while it fits.
    """
    L = np.asarray(L, np.float64)
    D = np.asarray(D, np.float64)
    bits = np.asarray(cand_bits, np.int64)
    N, C = D.shape
    assert L.shape == (N,) and bits.size == C and np.all(np.diff(bits) > 0)
    n_piv = int(round(pivot_frac * N))
    risk = L * D[:, -1]
    order = sorted(range(N), key=lambda u: (-risk[u], u))
    pivot = np.zeros(N, bool)
    pivot[order[:n_piv]] = True
    budget = nominal * N - PIVOT_BITS * n_piv
    rest = np.nonzero(~pivot)[0]
    used = int(bits[0]) * rest.size
    if used > budget:
        raise ValueError(f"budget of {nominal} bits per unit cannot hold {n_piv} pivots and the narrowest candidates")
    cost = L[:, None] * D
    choice = np.zeros(N, np.int64)
    hulls = {}
    heap = []
    for u in rest:
        h = _hull(bits, cost[u])
        hulls[u] = h
        if len(h) > 1:
            a, b = h[0], h[1]
            heapq.heappush(heap, (-(cost[u, a] - cost[u, b]) / (bits[b] - bits[a]), int(u), 1))
    while heap:
        _, u, pos = heapq.heappop(heap)
        h = hulls[u]
        a, b = h[pos - 1], h[pos]
        step = int(bits[b] - bits[a])
        if used + step > budget:
            continue
        used += step
        choice[u] = b
        if pos + 1 < len(h):
            c = h[pos + 1]
            heapq.heappush(heap, (-(cost[u, b] - cost[u, c]) / (bits[c] - bits[b]), u, pos + 1))
    kinds = bits[choice].astype(np.uint8)
    kinds[pivot] = synth.FP16
    return kinds, pivot


def row_impact(q, k, beta, gate, head: bool):
    """Coefficient of row i of the state stored before a step in that step's
    readout: o_t = S_t^T q_t with S_t = A_t S_{t-1} + beta_t k_t v_t^T and
    A_t = (I - beta_t k_t k_t^T) D_t, so d o_t / d S_{t-1}[i, j] = (A_t^T q_t)_i
    for every column j, = d_i (q_i - beta k_i (k . q)) (Tutorial §三: a row's
    impact is what an error stored in it contributes to the readout; Review
    (singularity-lens), row paragraph: from the state-update transform and the
    query).  q, k: [..., 128]; beta: [...]; gate: [...] (a scalar d per head,
    head=True) or [..., 128] (diagonal d_i).  Torch tensors, any device."""
    kq = (k * q).sum(dim=-1, keepdim=True)
    coef = q - beta[..., None] * k * kq
    return coef * (gate[..., None] if head else gate)


def _steps(cc: CalibConfig, cfg, tables, T):
    from . import workload
    for t in range(T):
        yield t, workload.step_inputs(cfg, tables, t)


def calibrate(cc: CalibConfig, device: str = "cuda") -> dict:
    """Steps 1-6 on the device path; returns the tables and the statistics."""
    import torch
    from . import workload

    cfg = cc.synth_config()
    tables = synth.static_tables(cfg)
    B, H, Dm = cc.n_seq, cc.H, qdr.DIM
    head = cc.unit == synth.UNIT_HEAD
    dev = torch.device(device)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    f32 = workload.fp32_pool(cfg, B)
    f32.qdr_slot_reset(slots)
    o = torch.empty((B, H, Dm), dtype=torch.float32, device=dev)
    sample_at = sorted({max(1, int(round(f * cc.T))) for f in cc.samples})
    samples = []
    ell_sum = torch.zeros(H if head else (H, Dm), dtype=torch.float64, device=dev)
    om_sum = torch.zeros((H, Dm), dtype=torch.float64, device=dev)
    n_om = 0
    t0 = time.perf_counter()
    for t, (q, k, v, beta, gate) in _steps(cc, cfg, tables, cc.T):
        g64 = gate.double()
        ell_sum += g64.log().sum(dim=0)
        if t > 0:   # the state stored after step t-1 is read out through step t's transform
            om_sum += row_impact(q.double(), k.double(), beta.double(), g64, head).square().sum(dim=0)
            n_om += B
        f32.qdr_decode_step(slots, q, k, v, beta, gate, o)
        if t + 1 in sample_at:
            S = torch.empty((B, H, Dm, Dm), dtype=torch.float32, device=dev)
            f32.qdr_unpack(slots, S)
            samples.append(S)
    if f32.qdr_poll_device_error():
        raise RuntimeError("device error word set during calibration")
    f32.close()
    ell = (ell_sum / (B * cc.T)).cpu().numpy()
    om = (om_sum / max(n_om, 1)).cpu().numpy()
    om = om / om.mean(axis=1, keepdims=True)
    omega = np.maximum(om, 1e-3).astype(np.float32)
    L = lifetime_weight(ell.reshape(-1), cc.horizon)
    cands = CANDIDATES[cc.nominal]
    Dist = np.empty((cc.n_units, len(cands)))
    w = torch.from_numpy(omega.astype(np.float64)).to(dev)
    for c, b in enumerate(cands):
        pool = qdr.Pool(B, H, np.full(cc.n_units, b, np.uint8), omega, unit=cc.unit, gate=cfg.gate,
                        scale_mode=qdr.SCALE_DUAL, fit_iters=cc.fit_iters)
        acc = torch.zeros((H, Dm), dtype=torch.float64, device=dev)
        R = torch.empty((B, H, Dm, Dm), dtype=torch.float32, device=dev)
        for S in samples:
            pool.qdr_pack(slots, S)
            pool.qdr_unpack(slots, R)
            acc += (R.double() - S.double()).square().sum(dim=(0, 3))    # [H, 128] rows
        if pool.qdr_poll_device_error():
            raise RuntimeError("device error word set while measuring distortion")
        pool.close()
        acc /= B * len(samples)
        if head:
            Dist[:, c] = ((acc * w).sum(dim=1) / (Dm * Dm)).cpu().numpy()
        else:
            Dist[:, c] = (acc / Dm).reshape(-1).cpu().numpy()
    kinds, pivot = allocate(L, Dist, cands, cc.nominal, cc.pivot_frac)
    return {"kinds": kinds, "omega": omega, "pivot": pivot, "ell": ell.reshape(-1), "L": L,
            "D": Dist, "candidates": np.asarray(cands), "calib_s": time.perf_counter() - t0,
            "synth_tables": tables}


def evaluate(cc: CalibConfig, allocations: dict, T: int | None = None, device: str = "cuda") -> dict:
    """Readout error of each allocation against the unquantised delta rule on
    held-out sequences (other seeds, same gates and outlier structure):
    sum ||o - o_fp32||^2 / sum ||o_fp32||^2 over all steps, sequences, heads.
    allocations: name -> (kinds, omega)."""
    import torch
    from . import workload

    cfg = cc.synth_config(held_out=True)
    tables = synth.static_tables(cc.synth_config())     # the calibrated units' gates and outliers
    B, H, Dm = cc.n_seq, cc.H, qdr.DIM
    dev = torch.device(device)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    ref = workload.fp32_pool(cfg, B)
    pools = {n: qdr.Pool(B, H, kd, om, unit=cc.unit, gate=cfg.gate, scale_mode=qdr.SCALE_DUAL,
                         fit_iters=cc.fit_iters) for n, (kd, om) in allocations.items()}
    for p in [ref, *pools.values()]:
        p.qdr_slot_reset(slots)
    o_ref = torch.empty((B, H, Dm), dtype=torch.float32, device=dev)
    o = torch.empty_like(o_ref)
    num = {n: 0.0 for n in pools}
    den = 0.0
    for t in range(T or cc.T):
        q, k, v, beta, gate = workload.step_inputs(cfg, tables, t)
        ref.qdr_decode_step(slots, q, k, v, beta, gate, o_ref)
        den += float(o_ref.double().square().sum())
        for n, p in pools.items():
            p.qdr_decode_step(slots, q, k, v, beta, gate, o)
            num[n] += float((o.double() - o_ref.double()).square().sum())
    out = {}
    for n, p in pools.items():
        if p.qdr_poll_device_error():
            raise RuntimeError("device error word set during evaluation")
        out[n] = {"rel_readout_sq_error": num[n] / den, "bits_per_value": p.bits_per_value,
                  "mean_code_bits": float(np.mean(allocations[n][0].astype(np.float64)))}
        p.close()
    ref.close()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description="offline calibration and bit allocation")
    ap.add_argument("--unit", choices=("head", "row"), default="head")
    ap.add_argument("--H", type=int, default=None)
    ap.add_argument("--n-seq", type=int, default=8)
    ap.add_argument("--T", type=int, default=256)
    ap.add_argument("--nominal", type=int, choices=(4, 6), default=None)
    ap.add_argument("--pivot-frac", type=float, default=None)
    ap.add_argument("--horizon", type=int, default=2048)
    ap.add_argument("--fit-iters", type=int, default=0, help="column-factor refits of the quantised pools")
    ap.add_argument("--out", default=None, help="write kinds, omega and the statistics to this .npz")
    a = ap.parse_args(argv)
    head = a.unit == "head"
    cc = CalibConfig(unit=synth.UNIT_HEAD if head else synth.UNIT_ROW,
                     H=a.H or (2304 if head else 1536), n_seq=a.n_seq, T=a.T,
                     nominal=a.nominal or (6 if head else 4),
                     pivot_frac=a.pivot_frac if a.pivot_frac is not None else (0.0139 if head else 0.01),
                     horizon=a.horizon, fit_iters=a.fit_iters)
    r = calibrate(cc)
    if a.out:
        np.savez(a.out, kinds=r["kinds"], omega=r["omega"], pivot=r["pivot"], ell=r["ell"], L=r["L"],
                 D=r["D"], candidates=r["candidates"])
    # the same budget spread uniformly (the nominal width everywhere, no pivots)
    uniform = np.full(cc.n_units, cc.nominal, np.uint8)
    ev = evaluate(cc, {"calibrated": (r["kinds"], r["omega"]),
                       "uniform_nominal_same_omega": (uniform, r["omega"]),
                       "uniform_nominal_omega1": (uniform, np.ones_like(r["omega"]))})
    kinds, cnt = np.unique(r["kinds"], return_counts=True)
    print(json.dumps({
        "calibration": "lifetime-aware allocation + row impact", "unit": a.unit, "units": cc.n_units,
        "heads": cc.H, "sequences": cc.n_seq, "steps": cc.T, "nominal_bits": cc.nominal,
        "candidates": list(CANDIDATES[cc.nominal]), "fit_iters": cc.fit_iters, "pivots": int(r["pivot"].sum()),
        "kind_counts": {int(k): int(c) for k, c in zip(kinds, cnt)},
        "mean_code_bits": float(np.mean(r["kinds"].astype(np.float64))), "calib_s": r["calib_s"],
        "held_out_eval": ev, "data": "synthetic"}), flush=True)


if __name__ == "__main__":
    sys.exit(main())
