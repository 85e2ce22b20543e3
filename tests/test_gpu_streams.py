"""The fused step on a caller's own stream and under HIP graph capture.

A whole-head pool with FP16 heads runs its FP16 launch on a stream of its own,
forked from the caller's stream and joined back to it by events.  These tests
check that this ordering holds where the caller relies on it:
  * on a non-default stream, work queued on that stream right after the step
    (a copy of o) sees the finished step, with no host synchronisation in
    between, and the stored state equals that of the step on the default
    stream;
  * captured into a graph and replayed, each replay equals one eager step on an
    identical pool (o and every stored byte), with eager work and
    synchronisations between the replays.
"""
import numpy as np
import pytest

from test_gpu_parity import D, random_inputs, row_kinds, t_
from quantized_delta_rule_decode_amd import qdr, synth

pytestmark = pytest.mark.gpu

KINDS = np.array([16, 8, 6, 4, 16, 2], np.uint8)


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "device tests need a HIP GPU"
    qdr.load()
    return torch


def packed_pool(torch, seed, n, unit="head"):
    """A packed pool: whole heads of KINDS (FP16 heads on the pool's second
    stream), or 3 row-unit heads with FP32 rows (a launch that raises the
    kernel's dynamic LDS limit)."""
    if unit == "head":
        kinds, H, u, gate, fp16 = KINDS, KINDS.size, qdr.UNIT_HEAD, qdr.GATE_SCALAR, None
    else:
        H = 3
        kinds, u, gate = row_kinds("fp32_rows", H, 7), qdr.UNIT_ROW, qdr.GATE_DIAG
        fp16 = kinds.reshape(H, D) == 16
    omega = np.random.default_rng(3).lognormal(0, 1, (H, D)).astype(np.float32)
    p = qdr.Pool(n, H, kinds, omega, unit=u, gate=gate)
    # ordinary (outlier but finite) states: several steps of the degenerate
    # edge states of the single-step tests overflow to inf/NaN
    S = synth.random_state(seed, n, H)
    if fp16 is not None:
        S = np.where(fp16[None, :, :, None], np.clip(S, -6e4, 6e4), S).astype(np.float32)
    p.qdr_pack(t_(torch, np.arange(n, dtype=np.int32)), t_(torch, S))
    torch.cuda.synchronize()
    return p


def test_step_on_user_stream(torch_dev):
    torch = torch_dev
    n, H = 4, KINDS.size
    ref = packed_pool(torch, 21, n)
    dev = packed_pool(torch, 21, n)
    slots = t_(torch, np.array([2, 0, 3, 1], np.int32))
    inputs = [t_(torch, x) for x in random_inputs(22, n, H, False)]
    o_ref = torch.empty((n, H, D), dtype=torch.float32, device="cuda")
    ref.qdr_decode_step(slots, *inputs, o_ref)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        side.wait_stream(torch.cuda.default_stream())
        o = torch.full((n, H, D), 5.0, dtype=torch.float32, device="cuda")
        dev.qdr_decode_step(slots, *inputs, o)
        o_copy = o.clone()            # queued on the same stream, no host sync
    side.synchronize()
    assert torch.equal(o_copy, o_ref)
    for s in range(n):
        assert np.array_equal(dev.qdr_read_raw(s), ref.qdr_read_raw(s))
    assert dev.qdr_poll_device_error() == 0


@pytest.mark.parametrize("unit", ["head", "row"])
def test_step_graph_replay(torch_dev, unit):
    torch = torch_dev
    n = 5
    eager = packed_pool(torch, 31, n, unit)
    graphed = packed_pool(torch, 31, n, unit)
    H, diag = graphed.num_heads, unit == "row"
    slots = t_(torch, np.array([4, 1, -1, 0, 2], np.int32))
    # static inputs, refilled in place before each replay
    q, k, v, beta, gate = [t_(torch, x) for x in random_inputs(32, n, H, diag)]
    o_g = torch.zeros((n, H, D), dtype=torch.float32, device="cuda")
    o_e = torch.zeros_like(o_g)

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            graphed.qdr_decode_step(slots, q, k, v, beta, gate, o_g)
    torch.cuda.synchronize()
    # capture enqueues nothing: both pools still hold the packed state
    for s in range(n):
        assert np.array_equal(graphed.qdr_read_raw(s), eager.qdr_read_raw(s))

    for it in range(4):
        new = random_inputs(40 + it, n, H, diag)
        for dst, src in zip((q, k, v, beta, gate), new):
            dst.copy_(torch.from_numpy(src).cuda())
        torch.cuda.synchronize()
        g.replay()
        eager.qdr_decode_step(slots, q, k, v, beta, gate, o_e)
        torch.cuda.synchronize()
        assert torch.isfinite(o_e).all()
        assert torch.equal(o_g, o_e), f"replay {it}: o differs"
        for s in range(n):
            assert np.array_equal(graphed.qdr_read_raw(s), eager.qdr_read_raw(s)), f"replay {it}: slot {s}"
        # eager work of the program's own between replays
        o_g.add_(0.0)
    assert graphed.qdr_poll_device_error() == 0 and eager.qdr_poll_device_error() == 0
