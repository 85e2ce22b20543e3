"""Benchmark of the fused quantized delta-rule decode step on one MI355X.

Workload (default): the full GDN pool -- B = 512 requests x 2304 heads of
128 x 128 states, nominal 6-bit (46 FP16 pivot heads, 691 INT8, 991 INT6,
576 INT4; mean 6.30 code bits), dual-axis scales, warm state from 256 FP32
delta-rule steps, about 15 GB of packed codes resident in HBM.  One "step" is
one qdr_decode_step over the whole pool: every (request, head) state is
restored, updated, read out, refitted, requantised and written back.

Prints one JSON line: state-update steps/s (requests x heads) and achieved HBM
GB/s from the algorithmic bytes, the roofline block, and the CPU oracle timed
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "state-update steps/s (requests x heads) at B=512, 6-bit; achieved HBM GB/s"


def algorithmic_bytes(cfg, tables, scale_bits: int = 32) -> int:
    """Bytes one step must move by the method's own accounting: every code
    (b bits per state value of its row, no layout padding) and every scale
    (scale_bits wide) read and written once, q/k/v, beta and the gate read,
    o written."""
    H = cfg.H
    kinds = np.asarray(tables["kinds"], np.int64)
    rows = np.repeat(kinds, 128).reshape(H, 128) if cfg.unit == 0 else kinds.reshape(H, 128)
    code = rows.sum(axis=1) * 128 // 8                       # bytes per head
    has_int = (rows <= 8).any(axis=1)
    scales = np.where(has_int, (2 if cfg.scale_mode == 0 else 1) * 128 * scale_bits // 8, 0)
    gate_bytes = 4 if cfg.gate == 0 else 4 * 128
    per_req = int((2 * code + 2 * scales).sum()) + H * (3 * 128 * 4 + 4 + gate_bytes + 128 * 4)
    return per_req * cfg.B


def measured_traffic(cid: int):
    """HBM bytes per step from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs (scaled by a plain-copy calibration), or None when the kernel source
    has changed since those counters were taken."""
    from quantized_delta_rule_decode_amd.build import device_source_hash
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
        sha = device_source_hash()
    except (OSError, ValueError):
        return None
    entry = rec.get(f"config{cid}")
    if rec.get("kernel_source_sha256_16") != sha or entry is None:
        return None
    return entry["fetch_bytes_per_step"] + entry["write_bytes_per_step"]


def cpu_baseline(cfg, tables, requests: int, threads: int):
    """The CPU oracle, as it stands, on `requests` requests x all heads."""
    from oracle import oracle as orc
    from quantized_delta_rule_decode_amd import synth
    P = orc.Pool(requests, cfg.H, tables["kinds"], tables["omega"], unit=cfg.unit,
                 gate=cfg.gate, scale_mode=cfg.scale_mode, fit_iters=cfg.fit_iters).alloc()
    slots = np.arange(requests, dtype=np.int32)
    P.pack(slots, synth.random_state(77, requests, cfg.H), threads=threads)
    sub = synth.Config(**{**cfg.__dict__, "B": requests, "device_inputs": False})
    ins = synth.step_inputs(sub, tables, 0)
    t0 = time.perf_counter()
    P.step(slots, *ins, threads=threads)
    dt = time.perf_counter() - t0
    return requests * cfg.H / dt, dt


def time_on_stream(fn, reps: int, warmup: int = 1) -> float:
    """Mean ms per call of fn() (device work on torch's current stream),
    HIP events recorded on that stream around `reps` calls."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def fp32_comparator(cfg, f32_pool, inputs, o, reps: int = 4):
    """The same decode step on an unquantised FP32 state pool of the same shape
    (the warm-up pool): the packed/FP32 speedup is the analogue of the pages'
    state-update speedup of the packed state over the FP32 state."""
    import torch
    B = cfg.B
    ident = torch.arange(B, dtype=torch.int32, device=o.device)
    ms = time_on_stream(lambda: f32_pool.qdr_decode_step(ident, *inputs, o), reps)
    per_head = 2 * 128 * 128 * 4 + 3 * 128 * 4 + 4 + (4 if cfg.gate == 0 else 4 * 128) + 128 * 4
    nbytes = per_head * B * cfg.H
    return {"ms_per_step": ms, "value": B * cfg.H / (ms * 1e-3), "unit": "state-update steps/s",
            "bytes_per_step": nbytes, "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
            "state": "fp32, 64 KiB per head, same kernel family (whole-head FP32 kind)"}


def fp32_trajectory_error(cid: int):
    """Error of the quantised decode trajectory against the unquantised delta
    rule on the same inputs: config `cid`'s pool and an FP32-kind pool start
    from the same state (the FP32 warm-up packed, or zero) and take the
    config's decode steps; relative L2 of the readouts over all steps and of
    the final states (the quantised one restored by qdr_unpack)."""
    import torch
    from quantized_delta_rule_decode_amd import qdr, synth, workload
    cfg = synth.CONFIGS[cid]
    tables = synth.static_tables(cfg)
    dev = torch.device("cuda")
    pool = workload.make_pool(cfg, tables)
    slots = torch.from_numpy(tables["slots"]).to(dev)
    ident = torch.arange(cfg.B, dtype=torch.int32, device=dev)
    if cfg.warmup > 0:
        ref = workload.warm_start(cfg, tables, pool, slots, cfg.warmup)
    else:
        ref = workload.fp32_pool(cfg, cfg.B)
        ref.qdr_slot_reset(ident)
        pool.qdr_slot_reset(slots)
    o = torch.empty((cfg.B, cfg.H, qdr.DIM), dtype=torch.float32, device=dev)
    o32 = torch.empty_like(o)
    num = den = 0.0
    for t in range(cfg.steps):
        q, k, v, beta, gate = workload.step_inputs(cfg, tables, t)
        pool.qdr_decode_step(slots, q, k, v, beta, gate, o)
        ref.qdr_decode_step(ident, q, k, v, beta, gate, o32)
        num += float((o.double() - o32.double()).square().sum())
        den += float(o32.double().square().sum())
    S = torch.empty((cfg.B, cfg.H, qdr.DIM, qdr.DIM), dtype=torch.float32, device=dev)
    S32 = torch.empty_like(S)
    pool.qdr_unpack(slots, S)
    ref.qdr_unpack(ident, S32)
    st = float((S.double() - S32.double()).norm() / S32.double().norm())
    assert pool.qdr_poll_device_error() == 0 and ref.qdr_poll_device_error() == 0
    pool.close()
    ref.close()
    return {"workload": cfg.name, "steps": cfg.steps, "o_rel_l2": (num / den) ** 0.5, "final_state_rel_l2": st}


def two_stream_split(pool, slots, inputs, o, fused_ms: float, reps: int = 5):
    """qdr_decode_step_split on the benchmark pool: how soon o is ready (the
    readout launches on their stream) and the whole split step, with and
    without a stand-in for downstream model work (an fp32 matmul chain) queued
    on the readout stream right after o, against the fused step followed by
    the same work on one stream."""
    import torch
    sr, sw = torch.cuda.Stream(), torch.cuda.Stream()
    a = torch.randn((4096, 4096), device="cuda")
    b = torch.randn((4096, 4096), device="cuda")

    def model_work(stream):
        with torch.cuda.stream(stream):
            c = a
            for _ in range(2):
                c = torch.mm(c, b)
        return c

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    def one(with_work: bool):
        torch.cuda.synchronize()
        ev[0].record(sr)
        pool.qdr_decode_step_split(slots, *inputs, o, sr, sw)
        ev[1].record(sr)
        if with_work:
            model_work(sr)
        sw.wait_stream(sr)
        ev[2].record(sw)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]), ev[0].elapsed_time(ev[2])

    one(True)
    ro = [one(False) for _ in range(reps)]
    wk = [one(True) for _ in range(reps)]
    cur = torch.cuda.current_stream()
    work_ms = time_on_stream(lambda: model_work(cur), reps)
    serial_ms = time_on_stream(lambda: (pool.qdr_decode_step(slots, *inputs, o), model_work(cur)), reps)
    return {"readout_ms": float(np.mean([r[0] for r in ro])), "split_total_ms": float(np.mean([r[1] for r in ro])),
            "fused_ms": fused_ms, "model_work": "2 x fp32 matmul 4096^3 on the readout stream after o",
            "model_work_ms": work_ms, "fused_then_work_ms": serial_ms,
            "split_with_work_ms": float(np.mean([r[1] for r in wk]))}


def compact_io(cfg, tables, pool, slots, inputs, fused_ms: float, reps: int = 5):
    """qdr_decode_step_bf16 on the benchmark pool: q, k, v and o in bfloat16
    (beta, gate fp32); its algorithmic bytes count 2 bytes per q/k/v/o value."""
    import torch
    q, k, v, beta, gate = inputs
    q16, k16, v16 = (x.to(torch.bfloat16) for x in (q, k, v))
    o16 = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    ms = time_on_stream(lambda: pool.qdr_decode_step_bf16(slots, q16, k16, v16, beta, gate, o16), reps)
    nbytes = algorithmic_bytes(cfg, tables) - cfg.B * cfg.H * 4 * 128 * 2
    return {"ms_per_step": ms, "value": cfg.B * cfg.H / (ms * 1e-3), "unit": "state-update steps/s",
            "algorithmic_bytes_per_step": nbytes, "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
            "speedup_over_fp32_io": fused_ms / ms}


def compact_scales(cfg, tables, pool, slots, inputs, o, fused_ms: float, reps: int = 5, chunk: int = 16):
    """The step on a pool that stores its scale factors as bfloat16: the
    benchmark pool's state is restored chunk by chunk (qdr_unpack) and packed
    into a 16-bit-scale pool of the same layout otherwise, then that pool's
    qdr_decode_step is timed on the same inputs."""
    import torch
    from quantized_delta_rule_decode_amd import qdr, workload
    p16 = workload.make_pool(cfg, tables, scale_bits=16)
    S = torch.empty((min(chunk, cfg.B), cfg.H, qdr.DIM, qdr.DIM), dtype=torch.float32, device=o.device)
    for i in range(0, cfg.B, chunk):
        s = slots[i:i + chunk]
        pool.qdr_unpack(s, S[:s.numel()])
        p16.qdr_pack(s, S[:s.numel()])
    del S
    torch.cuda.synchronize()
    ms = time_on_stream(lambda: p16.qdr_decode_step(slots, *inputs, o), reps)
    assert p16.qdr_poll_device_error() == 0
    nbytes = algorithmic_bytes(cfg, tables, scale_bits=16)
    out = {"ms_per_step": ms, "value": cfg.B * cfg.H / (ms * 1e-3), "unit": "state-update steps/s",
           "stored_bits_per_value": round(p16.bits_per_value, 3), "pool_bytes": p16.total_bytes,
           "algorithmic_bytes_per_step": nbytes, "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
           "speedup_over_fp32_scales": fused_ms / ms}
    p16.close()
    return out


def stream_reference(nbytes: int = 2 << 30, reps: int = 5):
    """HBM rate of a plain in-place streaming kernel on this GPU (torch add_ of
    an fp32 buffer: each byte read once and written once), for scale."""
    import torch
    x = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    ms = time_on_stream(lambda: x.add_(1.0), reps)
    del x
    return {"kernel": "torch.Tensor.add_ (in place, fp32)", "bytes": 2 * nbytes,
            "GBps": 2 * nbytes / (ms * 1e-3) / 1e9}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--fp32-warmup-steps", type=int, default=None,
                    help="FP32 delta-rule steps that build the warm state (default: the config's)")
    ap.add_argument("--cpu-requests", type=int, default=64,
                    help="requests in the oracle's timed sample (64 x 2304 heads: about 10 s on 16 cores)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp32-comparator", action="store_true",
                    help="skip timing the FP32-state pool of the warm-up")
    ap.add_argument("--no-split", action="store_true",
                    help="skip timing the two-stream step, the bfloat16-I/O step and the "
                         "bfloat16-scale pool")
    ap.add_argument("--no-trajectory-error", action="store_true",
                    help="skip the quantised-vs-FP32 trajectory error of the small configs")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n, "launches": 3}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the decode step has no "
              "cross-GPU term; heads or requests would shard across GPUs without communication",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_delta_rule_decode_amd import qdr, synth, workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = synth.CONFIGS[args.config]
    tables = synth.static_tables(cfg)
    dev = torch.device("cuda")
    t_setup = time.perf_counter()
    pool = workload.make_pool(cfg, tables)
    slots = torch.from_numpy(tables["slots"]).to(dev)
    warm = cfg.warmup if args.fp32_warmup_steps is None else args.fp32_warmup_steps
    q, k, v, beta, gate = workload.step_inputs(cfg, tables, 0, device=dev)
    o = torch.empty((cfg.B, cfg.H, 128), dtype=torch.float32, device=dev)
    fp32_cmp = None
    if warm > 0:
        f32 = workload.warm_start(cfg, tables, pool, slots, warm)
        if not args.no_fp32_comparator:
            fp32_cmp = fp32_comparator(cfg, f32, (q, k, v, beta, gate), o)
        f32.close()
        del f32
    else:
        pool.qdr_slot_reset(slots)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        pool.qdr_decode_step(slots, q, k, v, beta, gate, o)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        pool.qdr_decode_step(slots, q, k, v, beta, gate, o)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1) / args.steps
    assert pool.qdr_poll_device_error() == 0

    nbytes = algorithmic_bytes(cfg, tables)
    traffic = measured_traffic(cfg.cid)
    head_steps = cfg.B * cfg.H
    achieved = nbytes / (gpu_ms * 1e-3) / 1e9
    value = head_steps / (gpu_ms * 1e-3)

    split = None if args.no_split else two_stream_split(pool, slots, (q, k, v, beta, gate), o, gpu_ms)
    bf16_io = None if args.no_split else compact_io(cfg, tables, pool, slots, (q, k, v, beta, gate), gpu_ms)
    sc16 = None if args.no_split else compact_scales(cfg, tables, pool, slots, (q, k, v, beta, gate), o, gpu_ms)
    assert pool.qdr_poll_device_error() == 0
    stream = stream_reference()
    traj = None if args.no_trajectory_error else [fp32_trajectory_error(c) for c in (1, 2, 3)]
    cpu = None
    if not args.no_cpu_baseline:
        threads = min(os.cpu_count() or 1, 16)
        rate, dt = cpu_baseline(cfg, tables, args.cpu_requests, threads)
        cpu = {"value": rate, "unit": "state-update steps/s", "cores": threads, "kind": "oracle",
               "sample": f"{args.cpu_requests} requests x {cfg.H} heads, one step ({dt:.2f} s)"}

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "state-update steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": gpu_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "heads": cfg.H, "d_k": 128, "d_v": 128,
                   "mean_code_bits": round(float(np.mean(tables["kinds"])), 3),
                   "stored_bits_per_value": round(pool.bits_per_value, 3),
                   "fp32_warmup_steps": warm},
        "achieved_GBps": achieved,
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "unit_of_work": ("one qdr_decode_step: whole-head pools launch k_head_int over every "
                                      "integer head (the dominant kernel) and, on a second stream forked "
                                      "from and joined back to the caller's, one launch per float kind; "
                                      "row-unit pools launch k_rows once; achieved = algorithmic bytes per "
                                      "step / step time (HIP events on the caller's stream)"),
                     "traffic_over_algorithmic": None if traffic is None else traffic / nbytes,
                     "stream_reference": stream,
                     "frac_of_stream_reference": achieved / stream["GBps"]},
        "fp32_state_comparator": None if fp32_cmp is None else {
            **fp32_cmp, "speedup_packed_over_fp32": fp32_cmp["ms_per_step"] / gpu_ms},
        "two_stream_split": split,
        "bf16_io_step": bf16_io,
        "bf16_scales_step": sc16,
        "fp32_trajectory_error": traj,
        "cpu_baseline": cpu,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "setup_s": setup_s,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
