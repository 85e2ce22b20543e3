"""Decode step with bfloat16 q, k, v and o (qdr_decode_step_bf16).

The oracle steps on the bfloat16 inputs widened to fp32: the stored blocks
must match it exactly (same checks as the fp32 step) and o must be its readout
rounded to bfloat16 (elementwise within the bfloat16 rounding step).  On the
device, the bf16 step must equal the fp32 step on the widened inputs bit for
bit, up to the final rounding of o (nearest, ties to even).
"""
import numpy as np
import pytest

import parity
from test_gpu_parity import D, HEAD_KIND_SETS, edge_states, make_pair, random_inputs, row_kinds, t_
from quantized_delta_rule_decode_amd import qdr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "device tests need a HIP GPU"
    qdr.load()
    return torch


def widen(x16):
    """bfloat16 bit patterns (uint16) -> float32, exactly."""
    return (x16.astype(np.uint32) << 16).view(np.float32)


def round_bf16(x):
    """float32 -> bfloat16 bit patterns, nearest, ties to even (finite x)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


CASES = [("head", "with_pivots", 0), ("head", "int_all", 1), ("head", "fp32", 0), ("row", "kda_mix", 1)]


@pytest.mark.parametrize("sb", [32, 16])
@pytest.mark.parametrize("unit,name,gate", CASES)
def test_bf16_step_parity(torch_dev, orc, unit, name, gate, sb):
    torch = torch_dev
    if unit == "head":
        kinds = np.array(HEAD_KIND_SETS[name], np.uint8)
        H, u, fp16 = kinds.size, 0, None
    else:
        H, u = 3, 1
        kinds = row_kinds(name, H, 7)
        fp16 = kinds.reshape(H, D) == 16
    omega = np.random.default_rng(3).lognormal(0, 1, (H, D)).astype(np.float32)
    dev, ref = make_pair(orc, 6, kinds, omega, unit=u, gate=gate, sb=sb)
    twin = qdr.Pool(6, H, kinds, omega, unit=u, gate=gate, scale_bits=sb)   # fp32-I/O step on the widened inputs
    S = edge_states(23, 6, H, fp16)
    all_slots = np.arange(6, dtype=np.int32)
    for p in (dev, twin):
        p.qdr_pack(t_(torch, all_slots), t_(torch, S))
    ref.pack(all_slots, S)
    slots = np.array([4, -1, 0, 5, 2], np.int32)
    for step in range(2):
        print(f"bf16 {unit} {name} gate={gate} sb={sb} step {step}", flush=True)
        q, k, v, beta, g = random_inputs(50 + step, slots.size, H, gate == 1)
        q16, k16, v16 = (round_bf16(x) for x in (q, k, v))
        wq, wk, wv = (widen(x) for x in (q16, k16, v16))
        inputs = (wq, wk, wv, beta, g)
        prev = ref.mem.copy()
        o16 = torch.zeros((slots.size, H, D), dtype=torch.bfloat16, device="cuda")
        bf = [torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16) for x in (q16, k16, v16)]
        dev.qdr_decode_step_bf16(t_(torch, slots), *bf, t_(torch, beta), t_(torch, g), o16)
        o32 = torch.zeros((slots.size, H, D), dtype=torch.float32, device="cuda")
        twin.qdr_decode_step(t_(torch, slots), *(t_(torch, x) for x in inputs), o32)
        o_ref, bad = ref.step(slots, *inputs, threads=8)
        torch.cuda.synchronize()
        o_dev16 = o16.view(torch.int16).cpu().numpy().view(np.uint16)
        # device: the bf16 step is the fp32 step on the widened inputs, o rounded
        assert np.array_equal(o_dev16, round_bf16(o32.cpu().numpy())), "o differs from the rounded fp32 readout"
        for s in range(6):
            assert np.array_equal(dev.qdr_read_raw(s), twin.qdr_read_raw(s)), f"slot {s} differs from the fp32 step"
        # oracle: blocks as in the fp32 parity tests, o within one bfloat16 rounding
        rep = parity.StepReport()
        parity.compare_pool(orc, ref, dev, slots, parity.step_state_fn(orc, ref, prev, slots, inputs), rep)
        parity.assert_step_ok(rep, f"bf16 {unit} {name} gate={gate} sb={sb} step {step}")
        o_dev = widen(o_dev16)
        assert np.all(np.abs(o_dev - o_ref) <= 2.0 ** -8 * np.abs(o_ref) + 1e-38)
        assert np.linalg.norm(o_dev - o_ref) <= 2.0 ** -8 * np.linalg.norm(o_ref)
        assert bad == 0 and np.all(o_dev16[1] == 0)
    assert dev.qdr_poll_device_error() == 0
