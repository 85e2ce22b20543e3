"""The two-stream step (qdr_decode_step_split) on the device.

Readout-first launches on one stream, the write-back on a second stream
ordered after it: o and the stored state must equal the oracle's step (the
same checks as the fused step's parity tests), and must be bit-identical to
the fused qdr_decode_step on the device, over several consecutive steps
issued without host synchronisation (the library orders each call after the
previous write-back).
"""
import numpy as np
import pytest

import parity
from test_gpu_parity import (D, HEAD_KIND_SETS, edge_states, make_pair, random_inputs, row_kinds, t_)
from quantized_delta_rule_decode_amd import qdr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "device tests need a HIP GPU"
    qdr.load()
    return torch


def split_step_pair(torch, orc, dev, ref, slots, inputs, sr, sw, threads=8):
    prev = ref.mem.copy()
    dev_in = [t_(torch, x) for x in inputs]
    o = torch.full((slots.size, dev.num_heads, D), 3.0, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    dev.qdr_decode_step_split(t_(torch, slots), *dev_in, o, sr, sw)
    sr.synchronize()               # o is complete once the readout stream is
    o_dev = o.cpu().numpy()
    o_ref, bad = ref.step(slots, *inputs, threads=threads)
    torch.cuda.synchronize()
    rep = parity.StepReport()
    parity.compare_o(o_dev, o_ref, rep, ref.last_o_mag)
    parity.compare_pool(orc, ref, dev, slots, parity.step_state_fn(orc, ref, prev, slots, inputs), rep)
    return rep, o_dev, bad


CASES = [("head", name, gate) for name in sorted(HEAD_KIND_SETS) for gate in (0, 1)] + \
        [("row", "kda_mix", 1), ("row", "fp32_rows", 0)]


@pytest.mark.parametrize("sb", [32, 16])
@pytest.mark.parametrize("unit,name,gate", CASES)
def test_split_step_parity(torch_dev, orc, unit, name, gate, sb):
    torch = torch_dev
    if unit == "head":
        kinds = np.array(HEAD_KIND_SETS[name], np.uint8)
        H, u = kinds.size, 0
        fp16 = None
    else:
        H, u = 3, 1
        kinds = row_kinds(name, H, 7)
        fp16 = kinds.reshape(H, D) == 16
    omega = np.random.default_rng(3).lognormal(0, 1, (H, D)).astype(np.float32)
    dev, ref = make_pair(orc, 6, kinds, omega, unit=u, gate=gate, sb=sb)
    S = edge_states(21, 6, H, fp16)
    all_slots = np.arange(6, dtype=np.int32)
    dev.qdr_pack(t_(torch, all_slots), t_(torch, S))
    ref.pack(all_slots, S)
    sr, sw = torch.cuda.Stream(), torch.cuda.Stream()
    slots = np.array([4, -1, 0, 5, 2], np.int32)
    for step in range(2):
        print(f"split {unit} {name} gate={gate} sb={sb} step {step}", flush=True)
        inputs = random_inputs(30 + step, slots.size, H, gate == 1)
        rep, o_dev, bad = split_step_pair(torch, orc, dev, ref, slots, inputs, sr, sw)
        parity.assert_step_ok(rep, f"split {unit} {name} gate={gate} sb={sb} step {step}")
        assert bad == 0 and np.all(o_dev[1] == 0)
    for s in (1, 3):   # untouched slots keep their bytes
        assert np.array_equal(dev.qdr_read_raw(s), ref.mem[s * ref.slot_stride:(s + 1) * ref.slot_stride])
    assert dev.qdr_poll_device_error() == 0


@pytest.mark.parametrize("sb", [32, 16])
@pytest.mark.parametrize("unit", ["head", "row"])
def test_split_equals_fused_without_host_sync(torch_dev, unit, sb):
    torch = torch_dev
    if unit == "head":
        kinds = np.array([16, 8, 6, 4, 2, 6, 8, 32], np.uint8)
        H, u = kinds.size, 0
        fp16 = None
    else:
        H, u = 4, 1
        kinds = row_kinds("kda_mix", H, 9)
        fp16 = kinds.reshape(H, D) == 16
    omega = np.random.default_rng(4).lognormal(0, 1, (H, D)).astype(np.float32)
    gate = 1 if unit == "row" else 0
    fused = qdr.Pool(8, H, kinds, omega, unit=u, gate=gate, scale_bits=sb)
    split = qdr.Pool(8, H, kinds, omega, unit=u, gate=gate, scale_bits=sb)
    S = t_(torch, edge_states(22, 8, H, fp16))
    all_slots = t_(torch, np.arange(8, dtype=np.int32))
    fused.qdr_pack(all_slots, S)
    split.qdr_pack(all_slots, S)
    torch.cuda.synchronize()
    sr, sw = torch.cuda.Stream(), torch.cuda.Stream()
    slots = t_(torch, np.array([7, 2, -1, 0, 5, 3], np.int32))
    steps = [tuple(t_(torch, x) for x in random_inputs(40 + t, 6, H, gate == 1)) for t in range(4)]
    o_f = [torch.empty((6, H, D), dtype=torch.float32, device="cuda") for _ in steps]
    o_s = [torch.empty((6, H, D), dtype=torch.float32, device="cuda") for _ in steps]
    torch.cuda.synchronize()
    for t, ins in enumerate(steps):      # no host synchronisation between the steps
        fused.qdr_decode_step(slots, *ins, o_f[t])
        split.qdr_decode_step_split(slots, *ins, o_s[t], sr, sw)
    torch.cuda.synchronize()
    for t in range(len(steps)):
        assert torch.equal(o_f[t].view(torch.int32), o_s[t].view(torch.int32)), f"o differs at step {t}"
    for s in range(8):
        assert np.array_equal(fused.qdr_read_raw(s), split.qdr_read_raw(s)), f"slot {s} differs"
    assert fused.qdr_poll_device_error() == 0 and split.qdr_poll_device_error() == 0
