"""Device-side workload assembly for the benchmark and the device tests.

Builds pools for the synthetic configurations of ``synth`` and brings them to
their starting state using only the library's own entry points:
  * zero state: qdr_slot_reset;
  * warm state: FP32-kind steps of the same decode kernel (the unquantised
    delta rule), then qdr_unpack of the FP32 pool and qdr_pack into the
    quantised pool.
"""
from __future__ import annotations

import numpy as np
import torch

from . import qdr, synth


def make_pool(cfg: synth.Config, tables: dict, **kw) -> qdr.Pool:
    kinds = tables["kinds"]
    return qdr.Pool(cfg.num_slots, cfg.H, kinds, tables["omega"], unit=cfg.unit, gate=cfg.gate,
                    scale_mode=cfg.scale_mode, fit_iters=cfg.fit_iters, **kw)


def fp32_pool(cfg: synth.Config, num_slots: int) -> qdr.Pool:
    return qdr.Pool(num_slots, cfg.H, np.full(cfg.H, qdr.K_FP32, np.uint8),
                    np.ones((cfg.H, qdr.DIM), np.float32), unit=qdr.UNIT_HEAD, gate=cfg.gate,
                    scale_mode=qdr.SCALE_DUAL)


def inputs_to_device(host_inputs, device="cuda"):
    return tuple(torch.from_numpy(np.ascontiguousarray(x)).to(device) for x in host_inputs)


def step_inputs(cfg, tables, step, warmup=False, device="cuda"):
    """Per-step inputs on the device (host PCG64 for small configs, Philox for large)."""
    if cfg.device_inputs:
        return synth.step_inputs_device(cfg, tables, step, device, warmup=warmup)
    return inputs_to_device(synth.step_inputs(cfg, tables, step, warmup=warmup), device)


def warm_start(cfg, tables, pool: qdr.Pool, slots: torch.Tensor, warmup_steps: int,
               on_step=None, chunk: int = 32):
    """Run `warmup_steps` FP32 decode steps from zero, then pack into `pool`.

    on_step(step, inputs) is called with each step's device inputs (the device
    tests copy sampled heads out of them for the CPU oracle).
    Returns the FP32 pool (caller may close it).
    """
    B = slots.numel()
    f32 = fp32_pool(cfg, B)
    ident = torch.arange(B, dtype=torch.int32, device=slots.device)
    f32.qdr_slot_reset(ident)
    o = torch.empty((B, cfg.H, qdr.DIM), dtype=torch.float32, device=slots.device)
    for t in range(warmup_steps):
        q, k, v, beta, gate = step_inputs(cfg, tables, t, warmup=True)
        if on_step is not None:
            on_step(t, (q, k, v, beta, gate))
        f32.qdr_decode_step(ident, q, k, v, beta, gate, o)
    dense = torch.empty((min(chunk, B), cfg.H, qdr.DIM, qdr.DIM), dtype=torch.float32,
                        device=slots.device)
    for s in range(0, B, chunk):
        n = min(chunk, B - s)
        f32.qdr_unpack(ident[s:s + n], dense[:n])
        pool.qdr_pack(slots[s:s + n].contiguous(), dense[:n])
    torch.cuda.synchronize()
    return f32
