"""Error paths of the C ABI on a device: every rejected call returns its
status before anything is enqueued, so it leaves the pool, the outputs and
the device memory as they were.  The pool is allocated, reused and reclaimed
within the request lifecycle of a server (Tutorial "STEPQuant：取代 KV cache
的状态，6-bit 量化精度不掉", §六), so these paths are part of the boundary.

  * QDR_DEBUG=1: a slot listed twice or outside [-1, num_slots) -> QDR_E_SLOT
    from the host-side check, no launch (pack and reset also refuse -1);
  * a pool larger than the device -> QDR_E_NOMEM, no device memory kept;
    caller memory too small -> QDR_E_NOMEM, misaligned -> QDR_E_INVAL;
  * B < 0 (and n < 0) -> QDR_E_INVAL; raw slot I/O with a wrong size ->
    QDR_E_INVAL, with a slot out of range -> QDR_E_SLOT.
"""
import ctypes

import numpy as np
import pytest

from quantized_delta_rule_decode_amd import qdr

pytestmark = pytest.mark.gpu
D = 128
E_INVAL, E_NOMEM, E_SLOT = -1, -2, -4


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "device tests need a HIP GPU"
    qdr.load()
    return torch


def small_pool(num_slots=4, kinds=(6, 8, 4)):
    H = len(kinds)
    return qdr.Pool(num_slots, H, np.array(kinds, np.uint8), np.ones((H, D), np.float32))


def inputs(torch, B, H):
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    q = torch.randn((B, H, D), generator=g, device="cuda")
    k = torch.nn.functional.normalize(torch.randn((B, H, D), generator=g, device="cuda"), dim=-1)
    v = torch.randn((B, H, D), generator=g, device="cuda")
    beta = torch.rand((B, H), generator=g, device="cuda")
    gate = torch.rand((B, H), generator=g, device="cuda")
    return q, k, v, beta, gate


def snapshot(pool):
    return [pool.qdr_read_raw(s) for s in range(pool.num_slots)]


@pytest.mark.parametrize("slots", [[0, 2, 0], [1, 4], [3, -2], [1, 2, 1, -1]])
def test_debug_slot_check_rejects_before_launch(torch_dev, monkeypatch, slots):
    torch = torch_dev
    pool = small_pool()
    pool.qdr_slot_reset(torch.arange(4, dtype=torch.int32, device="cuda"))
    before = snapshot(pool)
    st = torch.tensor(slots, dtype=torch.int32, device="cuda")
    B, H = st.numel(), pool.num_heads
    o = torch.full((B, H, D), 7.0, device="cuda")
    monkeypatch.setenv("QDR_DEBUG", "1")
    with pytest.raises(qdr.QdrError) as ei:
        pool.qdr_decode_step(st, *inputs(torch, B, H), o)
    assert ei.value.status == E_SLOT and "QDR_DEBUG" in str(ei.value)
    for call in (lambda: pool.qdr_pack(st, torch.zeros((B, H, D, D), device="cuda")),
                 lambda: pool.qdr_slot_reset(st)):
        with pytest.raises(qdr.QdrError) as ei:
            call()
        assert ei.value.status == E_SLOT
    torch.cuda.synchronize()
    assert torch.all(o == 7.0).item()
    assert pool.qdr_poll_device_error() == 0
    assert all(np.array_equal(a, b) for a, b in zip(snapshot(pool), before))
    pool.close()


def test_debug_slot_check_accepts_padding_and_distinct_slots(torch_dev, monkeypatch):
    torch = torch_dev
    pool = small_pool()
    pool.qdr_slot_reset(torch.arange(4, dtype=torch.int32, device="cuda"))
    monkeypatch.setenv("QDR_DEBUG", "1")
    st = torch.tensor([3, -1, 0], dtype=torch.int32, device="cuda")
    o = torch.full((3, pool.num_heads, D), 7.0, device="cuda")
    pool.qdr_decode_step(st, *inputs(torch, 3, pool.num_heads), o)
    torch.cuda.synchronize()
    assert torch.all(o[1] == 0).item() and not torch.any(o[0] == 7.0).item()
    with pytest.raises(qdr.QdrError) as ei:        # pack has no padding rows
        pool.qdr_pack(st, torch.zeros((3, pool.num_heads, D, D), device="cuda"))
    assert ei.value.status == E_SLOT
    assert pool.qdr_poll_device_error() == 0
    pool.close()


def test_oversized_pool_is_nomem_and_keeps_nothing(torch_dev):
    torch = torch_dev
    torch.cuda.synchronize()
    free0, total = torch.cuda.mem_get_info()
    H = 1024
    kinds = np.full(H, 8, np.uint8)
    need = qdr.qdr_pool_bytes(250_000, H, kinds, np.ones((H, D), np.float32))
    assert need > 4 * total
    with pytest.raises(qdr.QdrError) as ei:
        qdr.Pool(250_000, H, kinds, np.ones((H, D), np.float32))
    assert ei.value.status == E_NOMEM
    free1, _ = torch.cuda.mem_get_info()
    assert abs(free1 - free0) < (64 << 20), (free0, free1)
    # the device is still usable
    pool = small_pool()
    pool.qdr_slot_reset(torch.arange(4, dtype=torch.int32, device="cuda"))
    assert pool.qdr_poll_device_error() == 0
    pool.close()


def test_caller_memory_too_small_or_misaligned(torch_dev):
    torch = torch_dev
    kinds = np.array([6, 8], np.uint8)
    om = np.ones((2, D), np.float32)
    need = qdr.qdr_pool_bytes(3, 2, kinds, om)
    buf = torch.zeros(need + 512, dtype=torch.uint8, device="cuda")
    with pytest.raises(qdr.QdrError) as ei:
        qdr.Pool(3, 2, kinds, om, dev_mem=buf[:need - 256])
    assert ei.value.status == E_NOMEM
    with pytest.raises(qdr.QdrError) as ei:
        qdr.Pool(3, 2, kinds, om, dev_mem=buf[4:need + 4])
    assert ei.value.status == E_INVAL
    pool = qdr.Pool(3, 2, kinds, om, dev_mem=buf[:need])     # exactly enough, aligned
    pool.qdr_slot_reset(torch.arange(3, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert pool.base == buf.data_ptr() and buf[:need].any().item()
    pool.close()


def test_negative_sizes_and_raw_io_arguments(torch_dev):
    torch = torch_dev
    L = qdr.load()
    pool = small_pool()
    pool.qdr_slot_reset(torch.arange(4, dtype=torch.int32, device="cuda"))
    before = snapshot(pool)
    B, H = 2, pool.num_heads
    st = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    q, k, v, beta, gate = inputs(torch, B, H)
    o = torch.full((B, H, D), 7.0, device="cuda")
    q16, k16, v16, o16 = (x.to(torch.bfloat16) for x in (q, k, v, o))
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    s0 = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    h = pool._h
    assert L.qdr_decode_step(h, P(st), -1, P(q), P(k), P(v), P(beta), P(gate), P(o), s0) == E_INVAL
    assert L.qdr_decode_step_bf16(h, P(st), -3, P(q16), P(k16), P(v16), P(beta), P(gate), P(o16), s0) == E_INVAL
    assert L.qdr_decode_step_split(h, P(st), -1, P(q), P(k), P(v), P(beta), P(gate), P(o), s0, s0) == E_INVAL
    S = torch.zeros((B, H, D, D), device="cuda")
    assert L.qdr_pack(h, P(st), -1, P(S), s0) == E_INVAL
    assert L.qdr_unpack(h, P(st), -1, P(S), s0) == E_INVAL
    assert L.qdr_slot_reset(h, P(st), -2, s0) == E_INVAL
    assert b"must be >= 0" in L.qdr_last_error()
    # null tensors with B > 0
    assert L.qdr_decode_step(h, P(st), B, None, P(k), P(v), P(beta), P(gate), P(o), s0) == E_INVAL
    # raw slot I/O
    buf = np.zeros(pool.slot_stride, np.uint8)
    bp = buf.ctypes.data_as(ctypes.c_void_p)
    assert L.qdr_read_raw(h, 0, bp, pool.slot_stride - 1, s0) == E_INVAL
    assert L.qdr_write_raw(h, 0, bp, pool.slot_stride + 1, s0) == E_INVAL
    assert L.qdr_read_raw(h, 4, bp, pool.slot_stride, s0) == E_SLOT
    assert L.qdr_write_raw(h, -1, bp, pool.slot_stride, s0) == E_SLOT
    torch.cuda.synchronize()
    assert torch.all(o == 7.0).item()
    assert all(np.array_equal(a, b) for a, b in zip(snapshot(pool), before))
    assert pool.qdr_poll_device_error() == 0
    pool.close()


def test_nonfinite_inputs_stay_in_their_head(torch_dev):
    """NaN and infinity in the inputs are not guarded: they propagate through
    their own (request, head) only.  The same step on a twin pool with clean
    inputs gives identical bytes and readouts everywhere else."""
    torch = torch_dev
    kinds = (6, 8, 4, 16)
    pools = [small_pool(num_slots=3, kinds=kinds) for _ in range(2)]
    st = torch.tensor([2, 0, 1], dtype=torch.int32, device="cuda")
    B, H = 3, len(kinds)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    S = torch.randn((3, H, D, D), generator=g, device="cuda")
    for p in pools:
        p.qdr_pack(torch.arange(3, dtype=torch.int32, device="cuda"), S)
    clean = inputs(torch, B, H)
    dirty = [x.clone() for x in clean]
    dirty[2][1, 0, 5] = float("nan")       # v of request 1, head 0
    dirty[0][2, 3, 7] = float("inf")       # q of request 2, head 3 (readout only)
    dirty[1][0, 2, 9] = float("-inf")      # k of request 0, head 2
    hit = {(1, 0), (2, 3), (0, 2)}
    outs = []
    for p, ins in zip(pools, (clean, dirty)):
        o = torch.empty((B, H, D), device="cuda")
        p.qdr_decode_step(st, *ins, o)
        torch.cuda.synchronize()
        assert p.qdr_poll_device_error() == 0
        outs.append(o.cpu().numpy())
    slot_of = st.cpu().numpy()
    for b in range(B):
        a, c = pools[0].qdr_read_raw(int(slot_of[b])), pools[1].qdr_read_raw(int(slot_of[b]))
        for h in range(H):
            if (b, h) in hit:
                continue
            assert np.array_equal(outs[0][b, h], outs[1][b, h]), f"readout of request {b} head {h}"
            off, n = int(pools[0].head_off[h]), int(pools[0].head_bytes[h])
            if (b, h) != (2, 3):   # a non-finite q touches only the readout
                assert np.array_equal(a[off:off + n], c[off:off + n]), f"block of request {b} head {h}"
    # the head whose readout saw the infinite q still stores the clean block
    off, n = int(pools[0].head_off[3]), int(pools[0].head_bytes[3])
    assert np.array_equal(pools[0].qdr_read_raw(int(slot_of[2]))[off:off + n],
                          pools[1].qdr_read_raw(int(slot_of[2]))[off:off + n])
    assert not np.all(np.isfinite(outs[1][2, 3]))
    for p in pools:
        p.close()
