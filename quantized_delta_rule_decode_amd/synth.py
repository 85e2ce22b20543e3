"""Seeded synthetic workloads for the quantized delta-rule decode step.

This module only draws random inputs and static tables; it holds none of the
method's arithmetic.  Both the device library's tests/benchmark and the CPU
oracle consume what it produces.

Distributions (the pages' shapes; no model, dataset or calibration corpus is
available, so synthetic inputs stand in for model activations):
  * 128 x 128 states per head, 2304 heads per request for the large GDN pool,
    batches up to 512 (tutorial §二/§三, review (singularity-lens) throughput
    paragraph);
  * q, k ~ N(0, 1)^128, L2-normalised in float64 then rounded to float32,
    q then scaled by 1/sqrt(128); v ~ N(0, 1); beta ~ U(0, 1);
  * GDN gate alpha_t = exp(-g), g ~ U(1e-4, 0.5) per step, or a per-head
    constant 2^(-1/hl) with half-life hl ~ logU[1, 4096];
  * KDA gate: per-(head, key-row) constant 2^(-1/hl_i), hl_i ~ logU[1, 4096];
  * outlier variant: value columns scaled by sigma_j ~ lognormal(0, 1) per
    (head, column), 4 fixed key channels per head multiplied by 8 before
    normalising (row/column outliers, tutorial §三 Figure 2 discussion);
  * omega ~ lognormal(0, 1) per (head, key row);
  * kinds ranked by the lifetime proxy (longest half-life gets FP16, then
    INT8, ...), or a seeded permutation when no per-unit half-life exists.
Host streams use numpy PCG64; the two large pools draw per-step inputs on the
device with torch's Philox generator.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

INT2, INT4, INT6, INT8, FP16, FP32 = 2, 4, 6, 8, 16, 32
UNIT_HEAD, UNIT_ROW = 0, 1
GATE_SCALAR, GATE_DIAG = 0, 1
SCALE_DUAL, SCALE_ROW_ABSMAX = 0, 1
D = 128


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    B: int
    H: int
    num_slots: int
    unit: int
    gate: int
    scale_mode: int
    steps: int
    warmup: int            # FP32 warmup steps before packing (0: zero state)
    outliers: bool         # outlier-column / outlier-key generators
    gate_mode: str         # "per_step", "per_head", "per_row"
    # column fit: 0 the clip-free range; 1 plus the weighted least-squares
    # refit, the fit of the pools that hold ternary (INT2) rows: with the
    # clip-free range an INT2 code rounds [c/2, c) up to c at every step, and
    # long-lived INT2 rows grow without bound
    fit_iters: int = 0
    device_inputs: bool = False

    @property
    def seed(self) -> int:
        return 1000 * self.cid


CONFIGS = {
    1: Config(1, "single_head_int8_rowabsmax", 1, 1, 1, UNIT_HEAD, GATE_SCALAR,
              SCALE_ROW_ABSMAX, 64, 256, False, "per_step"),
    2: Config(2, "gdn_b32_h48_nominal6", 32, 48, 32, UNIT_HEAD, GATE_SCALAR,
              SCALE_DUAL, 1024, 0, True, "per_head"),
    3: Config(3, "kda_b128_h32_nominal4", 128, 32, 128, UNIT_ROW, GATE_DIAG,
              SCALE_DUAL, 256, 0, False, "per_row", fit_iters=1),
    4: Config(4, "gdn_pool_b512_h2304_nominal6", 512, 2304, 512, UNIT_HEAD,
              GATE_SCALAR, SCALE_DUAL, 1, 256, False, "per_step",
              device_inputs=True),
    5: Config(5, "kda_slots2561_b512_h1536_nominal4", 512, 1536, 5 * 512 + 1,
              UNIT_ROW, GATE_DIAG, SCALE_DUAL, 64, 0, True, "per_row",
              fit_iters=1, device_inputs=True),
}


def rng(cfg: Config, stream: int, step: int | None = None) -> np.random.Generator:
    key = [cfg.seed + stream] if step is None else [cfg.seed + stream, step]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


# ---------------------------------------------------------------- allocation
def _rank_to_kinds(halflife: np.ndarray, shares: list[tuple[int, int]]) -> np.ndarray:
    """Longest-lived units first get the widest kind.  shares: (kind, count)."""
    order = np.argsort(-halflife, kind="stable")
    kinds = np.empty(halflife.size, np.uint8)
    pos = 0
    for kind, count in shares:
        kinds[order[pos:pos + count]] = kind
        pos += count
    assert pos == halflife.size
    return kinds


def _row_shares(n: int) -> list[tuple[int, int]]:
    """Row-unit allocation: 1% FP16, 10% INT8, 19% INT6, 40% INT4, rest INT2."""
    c16 = int(round(0.01 * n))
    c8 = int(round(0.10 * n))
    c6 = int(round(0.19 * n))
    c4 = int(round(0.40 * n))
    return [(FP16, c16), (INT8, c8), (INT6, c6), (INT4, c4), (INT2, n - c16 - c8 - c6 - c4)]


def static_tables(cfg: Config) -> dict:
    """Kinds, omega, gates fixed across steps, outlier structure, slot map."""
    g = rng(cfg, 0)
    H = cfg.H
    t: dict = {}
    t["omega"] = g.lognormal(0.0, 1.0, size=(H, D)).astype(np.float32)
    if cfg.gate_mode == "per_head":
        hl = np.exp(g.uniform(0.0, math.log(4096.0), size=H))
        t["halflife"] = hl
        t["alpha_head"] = (2.0 ** (-1.0 / hl)).astype(np.float32)
    elif cfg.gate_mode == "per_row":
        hl = np.exp(g.uniform(0.0, math.log(4096.0), size=(H, D)))
        t["halflife"] = hl
        t["a_row"] = (2.0 ** (-1.0 / hl)).astype(np.float32)
    if cfg.outliers:
        t["sigma"] = g.lognormal(0.0, 1.0, size=(H, D)).astype(np.float64)
        t["k_outlier"] = np.stack([g.choice(D, size=4, replace=False) for _ in range(H)])
    # kinds
    if cfg.cid == 1:
        t["kinds"] = np.full(H, INT8, np.uint8)
    elif cfg.cid == 2:
        t["kinds"] = _rank_to_kinds(t["halflife"], [(FP16, 1), (INT8, 14), (INT6, 21), (INT4, 12)])
    elif cfg.cid == 4:
        base = np.array([FP16] * 46 + [INT8] * 691 + [INT6] * 991 + [INT4] * 576, np.uint8)
        t["kinds"] = base[g.permutation(H)]
    else:  # row units ranked over the whole pool
        hl = t["halflife"].reshape(-1)
        t["kinds"] = _rank_to_kinds(hl, _row_shares(hl.size))
    # slot map: distinct random slots for the (5B+1)-slot pool, identity otherwise
    if cfg.num_slots > cfg.B:
        t["slots"] = np.sort(g.choice(cfg.num_slots, size=cfg.B, replace=False)).astype(np.int32)
        t["slots"] = t["slots"][g.permutation(cfg.B)]
    else:
        t["slots"] = np.arange(cfg.B, dtype=np.int32)
    return t


def mean_code_bits(cfg: Config, tables: dict) -> float:
    return float(np.asarray(tables["kinds"], np.float64).mean())


# ---------------------------------------------------------------- per-step inputs
def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def step_inputs(cfg: Config, tables: dict, step: int, warmup: bool = False,
                requests: np.ndarray | None = None):
    """Host (numpy float32) inputs for one step.

    Returns q, k, v [B,H,128], beta [B,H], gate [B,H] (scalar) or [B,H,128].
    `requests` restricts generation to a subset of request rows (the draw is
    made for the full batch so every subset sees the same numbers).
    """
    g = rng(cfg, 2 if warmup else 1, step)
    B, H = cfg.B, cfg.H
    q = g.standard_normal((B, H, D))
    k = g.standard_normal((B, H, D))
    v = g.standard_normal((B, H, D))
    beta = g.uniform(0.0, 1.0, size=(B, H))
    gs = g.uniform(1e-4, 0.5, size=(B, H)) if cfg.gate_mode == "per_step" else None
    if cfg.outliers:
        idx = tables["k_outlier"]
        k[:, np.arange(H)[:, None], idx] *= 8.0
        v = v * tables["sigma"][None]
    q = _unit(q) / math.sqrt(D)
    k = _unit(k)
    if cfg.gate_mode == "per_step":
        gate = np.exp(-gs)
    elif cfg.gate_mode == "per_head":
        gate = np.broadcast_to(tables["alpha_head"][None, :], (B, H))
    else:
        gate = np.broadcast_to(tables["a_row"][None], (B, H, D))
    out = [np.ascontiguousarray(x, dtype=np.float32) for x in (q, k, v, beta, gate)]
    if requests is not None:
        out = [np.ascontiguousarray(x[requests]) for x in out]
    return tuple(out)


def step_inputs_device(cfg: Config, tables: dict, step: int, device, warmup: bool = False):
    """Device (torch float32) inputs for one step of a large pool (Philox)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed * 100003 + (2 if warmup else 1) * 7919 + step)
    B, H = cfg.B, cfg.H
    f64 = torch.float64
    q = torch.randn((B, H, D), generator=gen, device=device, dtype=f64)
    k = torch.randn((B, H, D), generator=gen, device=device, dtype=f64)
    v = torch.randn((B, H, D), generator=gen, device=device, dtype=f64)
    beta = torch.rand((B, H), generator=gen, device=device, dtype=f64)
    if cfg.outliers:
        sig = torch.as_tensor(tables["sigma"], device=device)
        mult = torch.ones((H, D), dtype=f64, device=device)
        idx = torch.as_tensor(tables["k_outlier"], device=device)
        mult.scatter_(1, idx, 8.0)
        k = k * mult[None]
        v = v * sig[None]
    q = q / torch.linalg.vector_norm(q, dim=-1, keepdim=True) / math.sqrt(D)
    k = k / torch.linalg.vector_norm(k, dim=-1, keepdim=True)
    if cfg.gate_mode == "per_step":
        gs = torch.rand((B, H), generator=gen, device=device, dtype=f64) * (0.5 - 1e-4) + 1e-4
        gate = torch.exp(-gs)
    elif cfg.gate_mode == "per_head":
        gate = torch.as_tensor(tables["alpha_head"], device=device).expand(B, H)
    else:
        gate = torch.as_tensor(tables["a_row"], device=device).expand(B, H, D)
    return tuple(x.to(torch.float32).contiguous() for x in (q, k, v, beta, gate))


def random_state(seed: int, n: int, H: int, scale_rows: bool = True) -> np.ndarray:
    """Dense fp32 test states [n,H,128,128] with row and column outliers."""
    g = np.random.Generator(np.random.PCG64(seed))
    S = g.standard_normal((n, H, D, D))
    if scale_rows:
        S *= g.lognormal(0.0, 1.0, size=(n, H, D, 1))
        S *= g.lognormal(0.0, 1.0, size=(n, H, 1, D))
    return S.astype(np.float32)
