"""Error-propagation study on the device path.

The pages motivate lifetime-aware allocation by a measurement: across the
2,304 recurrent heads of the GDN model, a head's gate half-life predicts how
much error a uniform INT6 state accumulates (Spearman rho about 0.80:
Tutorial §三 opening paragraph; Review (ai-trend), Results; the validation
paragraph of Review (singularity-lens): four sequences sharing their inputs
with the FP32 state, 2,046 updates, accumulated squared state error, rho 0.8004
on the GDN model and 0.8017 on KDA).  This module repeats that measurement
with synthetic inputs:

  * every head h has a constant scalar retention alpha_h = 2^(-1/hl_h) with
    half-life hl_h ~ logU[1, 4096] (the per-head gate of the synthetic
    generators), so alpha_h^hl_h = 1/2; by default the heads also differ in
    scale the way the generators' outlier variant makes them (lognormal
    value-column scales, four outlier key channels per head), so the half-life
    is not the only thing that varies between heads;
  * B request sequences of T decode steps share their inputs (q, k, v, beta,
    gate) between two pools that start from the zero state:
      - an FP32-kind pool (the unquantised delta rule), and
      - a uniform INT6 pool with per-key-row absmax scales (the pages'
        uniform baseline);
    both are advanced with qdr_decode_step, the device hot path;
  * after every step both states are read back (qdr_unpack; the INT6 state is
    the restored stored state) and the accumulated squared state error of
    head h is
        E_h = sum over sequences b and steps t of ||S_int6[b,h,t] - S_fp32[b,h,t]||_F^2;
  * rho = Spearman rank correlation of (hl_h, E_h) over heads.
The relative final error mean_b ||S_int6 - S_fp32||_F / ||S_fp32||_F is
reported next to it (it removes the growth of the state's own norm with the
half-life).

Run: python -m quantized_delta_rule_decode_amd.study [--H 2304 --B 4 --T 512]
prints one JSON line.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import sys
import time

import numpy as np

from . import qdr, synth


@dataclasses.dataclass(frozen=True)
class StudyConfig:
    H: int = 2304
    B: int = 4
    T: int = 512
    outliers: bool = True     # per-head value-column scales and outlier key channels
    seed_id: int = 9          # seeds of the synthetic generators (synth.Config.cid)

    def synth_config(self) -> synth.Config:
        # per-head constant gate, uniform row-absmax INT6, zero start
        return synth.Config(self.seed_id, f"error_study_h{self.H}_b{self.B}_t{self.T}", self.B, self.H,
                            self.B, synth.UNIT_HEAD, synth.GATE_SCALAR, synth.SCALE_ROW_ABSMAX,
                            self.T, 0, self.outliers, "per_head", device_inputs=self.H * self.B > 4096)


def study_tables(sc: StudyConfig) -> dict:
    """Static tables of the study: the generators' per-head half-lives and
    gates, every head INT6."""
    cfg = sc.synth_config()
    t = synth.static_tables(cfg)
    t["kinds"] = np.full(sc.H, synth.INT6, np.uint8)
    return t


def halflife(alpha) -> np.ndarray:
    """Half-life of a constant retention alpha in (0, 1): the t with alpha^t = 1/2."""
    a = np.asarray(alpha, np.float64)
    return np.log(0.5) / np.log(a)


def ranks(x) -> np.ndarray:
    """Ranks 1..n of x, ties given the mean of the ranks they span."""
    x = np.asarray(x, np.float64)
    order = np.argsort(x, kind="stable")
    r = np.empty(x.size, np.float64)
    xs = x[order]
    i = 0
    while i < x.size:
        j = i
        while j + 1 < x.size and xs[j + 1] == xs[i]:
            j += 1
        r[order[i:j + 1]] = 0.5 * (i + j) + 1.0
        i = j + 1
    return r


def spearman(x, y) -> float:
    """Spearman rank correlation: the Pearson correlation of the ranks."""
    rx, ry = ranks(x), ranks(y)
    rx -= rx.mean()
    ry -= ry.mean()
    den = math.sqrt(float(np.dot(rx, rx)) * float(np.dot(ry, ry)))
    return float(np.dot(rx, ry) / den) if den > 0 else float("nan")


def run(sc: StudyConfig, device: str = "cuda") -> dict:
    """The study on the device path; returns rho, the per-head half-lives and
    errors, and the device time per step of each pool."""
    import torch
    from . import workload

    cfg = sc.synth_config()
    tables = study_tables(sc)
    B, H = sc.B, sc.H
    dev = torch.device(device)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    omega = np.ones((H, qdr.DIM), np.float32)   # not read by row-absmax scales
    p6 = qdr.Pool(B, H, tables["kinds"], omega, unit=qdr.UNIT_HEAD, gate=qdr.GATE_SCALAR,
                  scale_mode=qdr.SCALE_ROW_ABSMAX)
    p32 = workload.fp32_pool(cfg, B)
    o = torch.empty((B, H, qdr.DIM), dtype=torch.float32, device=dev)
    S6 = torch.empty((B, H, qdr.DIM, qdr.DIM), dtype=torch.float32, device=dev)
    S32 = torch.empty_like(S6)
    acc = torch.zeros((B, H), dtype=torch.float64, device=dev)
    t0 = time.perf_counter()
    p6.qdr_slot_reset(slots)
    p32.qdr_slot_reset(slots)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ms6 = ms32 = 0.0
    for t in range(sc.T):
        q, k, v, beta, gate = workload.step_inputs(cfg, tables, t)
        ev[0].record(stream)
        p6.qdr_decode_step(slots, q, k, v, beta, gate, o)
        ev[1].record(stream)
        p32.qdr_decode_step(slots, q, k, v, beta, gate, o)
        ev[2].record(stream)
        p6.qdr_unpack(slots, S6)
        p32.qdr_unpack(slots, S32)
        acc += (S6.double() - S32.double()).square().sum(dim=(2, 3))
        ev[2].synchronize()
        ms6 += ev[0].elapsed_time(ev[1])
        ms32 += ev[1].elapsed_time(ev[2])
    if p6.qdr_poll_device_error() or p32.qdr_poll_device_error():
        raise RuntimeError("device error word set during the study")
    rel = ((S6.double() - S32.double()).flatten(2).norm(dim=2) / S32.double().flatten(2).norm(dim=2))
    acc_np, rel_np = acc.cpu().numpy(), rel.cpu().numpy()
    p6.close()
    p32.close()
    wall = time.perf_counter() - t0
    hl = halflife(tables["alpha_head"])   # of the float32 retention the steps applied
    E = acc_np.sum(axis=0)
    e_rel = rel_np.mean(axis=0)
    return {"rho": spearman(hl, E), "rho_relative_final": spearman(hl, e_rel), "halflife": hl,
            "sq_error": E, "sq_error_per_request": acc_np, "rel_error_final": e_rel,
            "ms_per_step_int6": ms6 / sc.T, "ms_per_step_fp32": ms32 / sc.T, "wall_s": wall}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--H", type=int, default=2304)
    ap.add_argument("--B", type=int, default=4)
    ap.add_argument("--T", type=int, default=512)
    ap.add_argument("--no-outliers", action="store_true", help="heads differ only in their gate")
    a = ap.parse_args(argv)
    sc = StudyConfig(a.H, a.B, a.T, outliers=not a.no_outliers)
    r = run(sc)
    e, hl = r["sq_error"], r["halflife"]
    q = np.quantile(hl, [0.25, 0.5, 0.75])
    bands = [(0, q[0]), (q[0], q[1]), (q[1], q[2]), (q[2], np.inf)]
    print(json.dumps({
        "study": "spearman(half-life, accumulated squared uniform-INT6 state error) over heads",
        "heads": sc.H, "outlier_heads": sc.outliers, "sequences": sc.B, "steps_per_sequence": sc.T, "updates": sc.B * sc.T,
        "rho": r["rho"], "rho_relative_final_error": r["rho_relative_final"],
        "mean_sq_error_by_halflife_quartile": [float(e[(hl >= lo) & (hl < hi)].mean()) for lo, hi in bands],
        "ms_per_step_int6_rowabsmax": r["ms_per_step_int6"], "ms_per_step_fp32": r["ms_per_step_fp32"],
        "wall_s": r["wall_s"], "data": "synthetic"}), flush=True)


if __name__ == "__main__":
    sys.exit(main())
