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


def algorithmic_bytes(cfg, tables, scale_bits: int = 32, integer_heads_only: bool = False) -> int:
    """Bytes one step must move by the method's own accounting: every code
    (b bits per state value of its row, no layout padding) and every scale
    (scale_bits wide) read and written once, q/k/v, beta and the gate read,
    o written.  integer_heads_only: only the head-steps of the dominant launch
    (whole-head pools: the integer heads, which k_head_int takes; row-unit
    pools: every head, all in the one k_rows launch)."""
    H = cfg.H
    kinds = np.asarray(tables["kinds"], np.int64)
    rows = np.repeat(kinds, 128).reshape(H, 128) if cfg.unit == 0 else kinds.reshape(H, 128)
    code = rows.sum(axis=1) * 128 // 8                       # bytes per head
    has_int = (rows <= 8).any(axis=1)
    scales = np.where(has_int, (2 if cfg.scale_mode == 0 else 1) * 128 * scale_bits // 8, 0)
    gate_bytes = 4 if cfg.gate == 0 else 4 * 128
    vec = 3 * 128 * 4 + 4 + gate_bytes + 128 * 4
    take = (rows <= 8).all(axis=1) if (integer_heads_only and cfg.unit == 0) else np.ones(H, bool)
    per_req = int((2 * code + 2 * scales + vec)[take].sum())
    return per_req * cfg.B


def dominant_kernel(cfg) -> str:
    """rocprofv3's name of the step's dominant launch (template arguments:
    mode, gate, scale mode, column fit)."""
    name = "k_head_int" if cfg.unit == 0 else "k_rows"
    return f"void qdr::{name}<0, {cfg.gate}, {cfg.scale_mode}, {1 if cfg.fit_iters else 0}>(qdr::LaunchArgs)"


def measured_traffic(cid: int, kernel: str | None = None):
    """HBM bytes per step from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs (scaled by the calibration of those counters): of the whole step, or
    of one kernel's launch.  None when the kernel sources have changed since
    those counters were taken, or nothing was recorded for the workload."""
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
    if kernel is None:
        return entry["fetch_bytes_per_step"] + entry["write_bytes_per_step"]
    k = entry.get("kernel_bytes", {}).get(kernel)
    return None if k is None else k["fetch"] + k["write"]


def cpu_baseline(cfg, tables, requests: int, threads: int, compare: bool = False):
    """The CPU oracle, as it stands, on `requests` requests x all heads.
    compare: also run the same step (same packed state, same inputs) through
    the library on a pool of those requests and report how the results agree:
    blocks byte for byte, the readout at relative L2."""
    from oracle import oracle as orc
    from quantized_delta_rule_decode_amd import synth
    P = orc.Pool(requests, cfg.H, tables["kinds"], tables["omega"], unit=cfg.unit,
                 gate=cfg.gate, scale_mode=cfg.scale_mode, fit_iters=cfg.fit_iters).alloc()
    slots = np.arange(requests, dtype=np.int32)
    S = synth.random_state(77, requests, cfg.H)
    P.pack(slots, S, threads=threads)
    sub = synth.Config(**{**cfg.__dict__, "B": requests, "device_inputs": False})
    ins = synth.step_inputs(sub, tables, 0)
    t0 = time.perf_counter()
    o_ref, _ = P.step(slots, *ins, threads=threads)
    dt = time.perf_counter() - t0
    parity = None
    if compare:
        import torch
        from quantized_delta_rule_decode_amd import qdr
        dev = qdr.Pool(requests, cfg.H, tables["kinds"], tables["omega"], unit=cfg.unit, gate=cfg.gate,
                       scale_mode=cfg.scale_mode, fit_iters=cfg.fit_iters)
        ds = torch.from_numpy(slots).cuda()
        dev.qdr_pack(ds, torch.from_numpy(S).cuda())
        o = torch.empty((requests, cfg.H, 128), dtype=torch.float32, device="cuda")
        dev.qdr_decode_step(ds, *(torch.from_numpy(np.ascontiguousarray(x)).cuda() for x in ins), o)
        torch.cuda.synchronize()
        same = sum(int(np.array_equal(dev.qdr_read_raw(i), P.mem[i * P.slot_stride:(i + 1) * P.slot_stride]))
                   for i in range(requests))
        od, orf = o.cpu().numpy().astype(np.float64), np.asarray(o_ref, np.float64)
        parity = {"requests": requests, "slots_byte_identical": same,
                  "o_rel_l2": float(np.linalg.norm(od - orf) / np.linalg.norm(orf))}
        dev.close()
    return requests * cfg.H / dt, dt, parity


def other_configs(cids=(1, 2, 3, 5), reps: int = 20):
    """The other workloads' own figures: config 1 (one head) as latency per
    step, configs 2 and 3 (cache-resident pools) as state-update steps/s,
    config 5 (the (5B+1)-slot KDA pool, 38.7 GB) as steps/s, achieved GB/s of
    its algorithmic bytes and the fraction of 8 TB/s.  Each pool starts from
    its own initial state (config 1: 256 FP32 steps then pack; the others:
    the zero state) and takes a few untimed steps before the timed ones; every
    step is one qdr_decode_step on the same inputs."""
    import torch
    from quantized_delta_rule_decode_amd import synth, workload
    out = {}
    for cid in cids:
        cfg = synth.CONFIGS[cid]
        tables = synth.static_tables(cfg)
        pool = workload.make_pool(cfg, tables)
        slots = torch.from_numpy(tables["slots"]).cuda()
        if cfg.warmup:
            workload.warm_start(cfg, tables, pool, slots, cfg.warmup).close()
        else:
            pool.qdr_slot_reset(slots)
        ins = workload.step_inputs(cfg, tables, 0)
        o = torch.empty((cfg.B, cfg.H, 128), dtype=torch.float32, device="cuda")
        ms = time_on_stream(lambda: pool.qdr_decode_step(slots, *ins, o), reps, warmup=5)
        assert pool.qdr_poll_device_error() == 0
        nbytes = algorithmic_bytes(cfg, tables)
        rec = {"workload": cfg.name, "B": cfg.B, "heads": cfg.H, "ms_per_step": ms,
               "state_update_steps_per_s": cfg.B * cfg.H / (ms * 1e-3),
               "algorithmic_bytes_per_step": nbytes, "timed_steps": reps}
        if cid == 1:
            rec["latency_us_per_step"] = ms * 1e3
        if cid == 5:
            gbps = nbytes / (ms * 1e-3) / 1e9
            rec.update({"achieved_GBps": gbps, "frac_of_peak_hbm": gbps / PEAK_HBM_GBPS,
                        "kernel": "k_rows (row units: per-key-row kinds)"})
        out[f"config{cid}"] = rec
        pool.close()
        del pool
        torch.cuda.synchronize()
    return out


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


def fp32_trajectory_error(cid: int, fit_iters: int | None = None):
    """Error of the quantised decode trajectory against the unquantised delta
    rule on the same inputs: config `cid`'s pool and an FP32-kind pool start
    from the same state (the FP32 warm-up packed, or zero) and take the
    config's decode steps; relative L2 of the readouts over all steps and of
    the final states (the quantised one restored by qdr_unpack).  fit_iters
    overrides the config's column fit (0: clip-free range, 1: least-squares
    refit)."""
    import dataclasses
    import torch
    from quantized_delta_rule_decode_amd import qdr, synth, workload
    cfg = synth.CONFIGS[cid]
    if fit_iters is not None:
        cfg = dataclasses.replace(cfg, fit_iters=fit_iters)
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
    return {"workload": cfg.name, "steps": cfg.steps, "column_fit": "least-squares refit" if cfg.fit_iters else "clip-free range",
            "o_rel_l2": (num / den) ** 0.5, "final_state_rel_l2": st}


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


def batch_sweep(cfg, tables, pool, slots, inputs, o, batches=(32, 64, 128, 256), reps: int = 10):
    """The same pool stepped for the first b requests only, for each b: the
    decode-step throughput over batch sizes (the pages time the whole step
    at batches from 32 to 512: Review (singularity-lens), throughput
    paragraph).  Every step is one qdr_decode_step on the same inputs."""
    import dataclasses
    out = []
    for b in batches:
        if b >= cfg.B:
            continue
        sub = dataclasses.replace(cfg, B=b)
        ins = tuple(x[:b] for x in inputs)
        ms = time_on_stream(lambda: pool.qdr_decode_step(slots[:b], *ins, o[:b]), reps, warmup=2)
        nbytes = algorithmic_bytes(sub, tables)
        out.append({"B": b, "ms_per_step": ms, "state_update_steps_per_s": b * cfg.H / (ms * 1e-3),
                    "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
                    "frac_of_peak_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS})
    return out


def clock_under_load(pool, slots, inputs, o, probes: int = 3):
    """The shader clock (qdr_clock_probe: one wave between two reads of the
    clock counter and of the 100 MHz counter) while idle, and while decode
    steps run: the probe goes on a second stream during every tenth-step
    batch.  A VALU-bound step's time scales with this clock, which the GPU
    lowers under a heavy load."""
    import torch
    from quantized_delta_rule_decode_amd import qdr
    out = torch.zeros(8, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()

    def mhz():
        t0, r0, t1, r1 = (int(x) for x in out[:4].cpu().tolist())
        return 100.0 * (t1 - t0) / (r1 - r0)

    qdr.qdr_clock_probe(out, 2000, side)
    torch.cuda.synchronize()
    idle = mhz()
    loaded = []
    for _ in range(probes):
        for i in range(10):
            pool.qdr_decode_step(slots, *inputs, o)
            if i == 3:
                qdr.qdr_clock_probe(out, 300, side)
        torch.cuda.synchronize()
        loaded.append(mhz())
    return {"idle_MHz": idle, "during_steps_MHz": loaded,
            "probe": "qdr_clock_probe on a second stream, one wave"}


def stream_reference(nbytes: int = 2 << 30, reps: int = 5):
    """HBM rate of a plain in-place streaming kernel on this GPU (torch add_ of
    an fp32 buffer: each byte read once and written once), for scale."""
    import torch
    x = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    ms = time_on_stream(lambda: x.add_(1.0), reps)
    del x
    return {"kernel": "torch.Tensor.add_ (in place, fp32)", "bytes": 2 * nbytes,
            "GBps": 2 * nbytes / (ms * 1e-3) / 1e9}


def calibration(kind: str, cid: int, launches: int = 3):
    """Three launches of a kernel whose HBM bytes are known; prints them as
    one JSON line.  rocprofv3's FETCH_SIZE / WRITE_SIZE per dispatch over
    these bytes gives the factor its readings are scaled by (one copy and one
    in-place pattern, and the decode step's own block loads and stores)."""
    import torch
    if kind in ("copy", "inplace"):
        n = 4 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src) if kind == "copy" else None
        for _ in range(launches):
            if kind == "copy":
                dst.copy_(src)
            else:
                src.add_(1.0)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": kind, "read_bytes": n, "write_bytes": n, "launches": launches,
                          "kernel": "torch copy_" if kind == "copy" else "torch add_ (in place)"}), flush=True)
        return
    from quantized_delta_rule_decode_amd import synth, workload
    cfg = synth.CONFIGS[cid]
    tables = synth.static_tables(cfg)
    B = 64
    pool = workload.fp32_pool(cfg, B)
    ident = torch.arange(B, dtype=torch.int32, device="cuda")
    pool.qdr_slot_reset(ident)
    sub = synth.Config(**{**cfg.__dict__, "B": B})
    q, k, v, beta, gate = workload.step_inputs(sub, tables, 0)
    o = torch.empty((B, cfg.H, 128), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    for _ in range(launches):
        pool.qdr_decode_step(ident, q, k, v, beta, gate, o)
    torch.cuda.synchronize()
    assert pool.qdr_poll_device_error() == 0
    heads = B * cfg.H
    block = 128 * 128 * 4
    vec_in = 3 * 128 * 4 + 4 + (4 if cfg.gate == 0 else 4 * 128)
    print(json.dumps({"calibration": kind, "workload": cfg.name, "requests": B, "heads": heads,
                      "read_bytes": heads * (block + vec_in), "write_bytes": heads * (block + 128 * 4),
                      "block_bytes_each_way": heads * block, "launches": launches,
                      "kernel": "k_head<32, ...> (FP32-kind decode step)"}), flush=True)
    pool.close()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--fit-iters", type=int, default=None, choices=(0, 1),
                    help="column fit of the timed pool: 0 the clip-free range, 1 plus the least-squares refit "
                         "(default: the workload's own)")
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
    ap.add_argument("--no-clock", action="store_true",
                    help="skip measuring the shader clock while idle and during decode steps")
    ap.add_argument("--no-batch-sweep", action="store_true",
                    help="skip timing the step on the first 32, 64, 128 and 256 requests of the pool")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip timing configs 1, 2, 3 and 5 next to the benchmark configuration")
    ap.add_argument("--cpu-requests-single", type=int, default=2,
                    help="requests in the single-threaded oracle sample (2 x 2304 heads: about 10 s)")
    ap.add_argument("--calibration", choices=("copy", "inplace", "fp32pool"), default=None,
                    help="only run a kernel of known HBM bytes (calibrates rocprofv3's byte counters): "
                         "copy = a 4 GiB device copy, inplace = torch add_ on 4 GiB (read, then written "
                         "in place), fp32pool = the decode step on an FP32-kind pool of 64 requests x "
                         "the config's heads (each 64 KiB block read and written back in place by the "
                         "step's own buffer loads and stores)")
    args = ap.parse_args()
    if args.calibration:
        calibration(args.calibration, args.config)
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
    if args.fit_iters is not None:
        import dataclasses
        cfg = dataclasses.replace(cfg, fit_iters=args.fit_iters)
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
    # one event between consecutive steps: the first and last bracket the K
    # timed steps (their mean is ms_per_step), the others give each step's
    # own time for the median, min and max
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    t0 = time.perf_counter()
    for i in range(args.steps):
        pool.qdr_decode_step(slots, q, k, v, beta, gate, o)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    assert pool.qdr_poll_device_error() == 0

    nbytes = algorithmic_bytes(cfg, tables)
    head_steps = cfg.B * cfg.H
    achieved_step = nbytes / (gpu_ms * 1e-3) / 1e9
    value = head_steps / (gpu_ms * 1e-3)
    # the roofline of the dominant launch: its own head-steps' bytes over its
    # duration, which is the step time (it is launched on the caller's stream
    # and spans the step; the float-kind launch runs inside it)
    kernel = dominant_kernel(cfg)
    kbytes = algorithmic_bytes(cfg, tables, integer_heads_only=True)
    achieved = kbytes / (gpu_ms * 1e-3) / 1e9
    traffic = measured_traffic(cfg.cid, kernel)

    split = None if args.no_split else two_stream_split(pool, slots, (q, k, v, beta, gate), o, gpu_ms)
    bf16_io = None if args.no_split else compact_io(cfg, tables, pool, slots, (q, k, v, beta, gate), gpu_ms)
    sc16 = None if args.no_split else compact_scales(cfg, tables, pool, slots, (q, k, v, beta, gate), o, gpu_ms)
    assert pool.qdr_poll_device_error() == 0
    stream = stream_reference()
    traj = None if args.no_trajectory_error else \
        [fp32_trajectory_error(1)] + [fp32_trajectory_error(c, f) for c in (2, 3) for f in (0, 1)]
    sweep = None if args.no_batch_sweep else batch_sweep(cfg, tables, pool, slots, (q, k, v, beta, gate), o)
    clock = None if args.no_clock else clock_under_load(pool, slots, (q, k, v, beta, gate), o)
    assert pool.qdr_poll_device_error() == 0
    others = None if args.no_other_configs else other_configs()
    cpu = None
    if not args.no_cpu_baseline:
        host_cores = os.cpu_count() or 1
        threads = min(host_cores, 16)
        rate, dt, par = cpu_baseline(cfg, tables, args.cpu_requests, threads, compare=True)
        rate1, dt1, _ = cpu_baseline(cfg, tables, args.cpu_requests_single, 1)
        cpu = {"value": rate, "unit": "state-update steps/s", "cores": threads, "kind": "oracle",
               "sample": f"{args.cpu_requests} requests x {cfg.H} heads, one step ({dt:.2f} s) on {threads} threads",
               "host_cores": host_cores,
               "parity_with_device": par,
               "single_thread": {"value": rate1, "unit": "state-update steps/s", "cores": 1,
                                 "sample": f"{args.cpu_requests_single} requests x {cfg.H} heads, one step "
                                           f"({dt1:.2f} s)"}}

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "state-update steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": gpu_ms,
        "ms_per_step_median": float(np.median(per_step)),
        "ms_per_step_min": per_step[0],
        "ms_per_step_max": per_step[-1],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "inputs": {"tables": f"numpy PCG64, SeedSequence([{cfg.seed} + stream])",
                   "step_inputs": ("torch Philox on the device, seed "
                                   f"{cfg.seed} * 100003 + 7919 + step" if cfg.device_inputs
                                   else f"numpy PCG64, SeedSequence([{cfg.seed} + stream, step])"),
                   "warm_state": f"{warm} FP32 decode steps from zero, then packed" if warm else "zero state"},
        "config": {"workload": cfg.name, "B": cfg.B, "heads": cfg.H, "d_k": 128, "d_v": 128,
                   "mean_code_bits": round(float(np.mean(tables["kinds"])), 3),
                   "stored_bits_per_value": round(pool.bits_per_value, 3),
                   "fp32_warmup_steps": warm},
        "achieved_GBps": achieved_step,
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic,
                     "kernel": kernel, "algorithmic_bytes_per_launch": kbytes,
                     "launch_ms": gpu_ms,
                     "whole_step": {"algorithmic_bytes": nbytes, "achieved": achieved_step,
                                    "frac": achieved_step / PEAK_HBM_GBPS},
                     "unit_of_work": ("one launch of the dominant kernel per decode step: whole-head pools "
                                      "launch k_head_int over every integer head and, on a second stream "
                                      "forked from and joined back to the caller's, one launch per float "
                                      "kind, which runs inside the integer launch's span; row-unit pools "
                                      "launch k_rows once.  achieved = the launch's algorithmic bytes (its "
                                      "head-steps x their bytes per head-step) / its duration, the step "
                                      "time of HIP events on the caller's stream, the launch's own stream; "
                                      "achieved_GBps at the top counts every head of the step"),
                     "traffic_over_algorithmic": None if traffic is None else traffic / kbytes,
                     "stream_reference": stream,
                     "frac_of_stream_reference": achieved_step / stream["GBps"]},
        "fp32_state_comparator": None if fp32_cmp is None else {
            **fp32_cmp, "speedup_packed_over_fp32": fp32_cmp["ms_per_step"] / gpu_ms},
        "two_stream_split": split,
        "bf16_io_step": bf16_io,
        "bf16_scales_step": sc16,
        "fp32_trajectory_error": traj,
        "batch_sweep": sweep,
        "shader_clock": clock,
        "other_configs": others,
        "cpu_baseline": cpu,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "setup_s": setup_s,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
