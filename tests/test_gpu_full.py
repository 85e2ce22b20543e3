"""Full-size device runs in the benchmark's launch configuration.

Config 4 is the benchmark's own launch: the 512 x 2304-head GDN pool, one
quantised decode step over every request.  Two checks: every head of eight
requests (0 and 511 among them) from a dense state generated on the host,
which both sides pack; the same for three requests under each step variant
the benchmark also times (bfloat16 factors, bfloat16 I/O, the two-launch
step); and sampled heads of the benchmark's own warm state (256 FP32 decode
steps, then pack).  Config 5 is the (5B+1)-slot KDA pool
with a random slot map, 64 decode steps from the zero state over all 512
requests, every head of one request per case checked at every step.  The
oracle gets the same seeded inputs (copied from the device generator) and
never reads a byte the device produced; unmapped slots stay untouched.
"""
import numpy as np
import pytest

from quantized_delta_rule_decode_amd import qdr, synth, workload

import parity

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "device tests need a HIP GPU"
    qdr.load()
    return torch


def pick_samples(kinds_per_head, B, H, per_kind=3, seed=0):
    g = np.random.default_rng(seed)
    out = [(0, 0), (B - 1, H - 1)]
    for kd in np.unique(kinds_per_head):
        hs = np.nonzero(kinds_per_head == kd)[0]
        for h in g.choice(hs, size=min(per_kind, hs.size), replace=False):
            out.append((int(g.integers(0, B)), int(h)))
    return sorted(set(out))


def host_slice(inputs, b, h):
    q, k, v, beta, gate = inputs
    gh = gate[b, h]
    return (q[b, h].cpu().numpy(), k[b, h].cpu().numpy(), v[b, h].cpu().numpy(),
            float(beta[b, h].item()),
            np.full(D, gh.item(), np.float32) if gh.dim() == 0 else gh.cpu().numpy())


def head_kinds(cfg, t, h):
    return np.full(D, t["kinds"][h], np.uint8) if cfg.unit == 0 else t["kinds"][h * D:(h + 1) * D]


def dev_block(pool, slot, h):
    raw = pool.qdr_read_raw(int(slot))
    off = int(pool.head_off[h])
    return raw[off: off + int(pool.head_bytes[h])]


def test_config4_full_pool_sampled(torch_dev, orc):
    torch = torch_dev
    cfg = synth.CONFIGS[4]
    t = synth.static_tables(cfg)
    samples = pick_samples(t["kinds"], cfg.B, cfg.H)
    pool = workload.make_pool(cfg, t)
    slots = torch.from_numpy(t["slots"]).cuda()
    warm_inputs = {s: [] for s in samples}

    def record(step, ins):
        for (b, h) in samples:
            warm_inputs[(b, h)].append(host_slice(ins, b, h))

    f32 = workload.warm_start(cfg, t, pool, slots, cfg.warmup, on_step=record)
    f32.close()
    ins = workload.step_inputs(cfg, t, 0)
    o = torch.empty((cfg.B, cfg.H, D), dtype=torch.float32, device="cuda")
    before = {s: dev_block(pool, t["slots"][s[0]], s[1]) for s in samples}
    pool.qdr_decode_step(slots, *ins, o)
    torch.cuda.synchronize()
    assert pool.qdr_poll_device_error() == 0
    k32 = np.full(D, 32, np.uint8)
    for (b, h) in samples:
        kinds = head_kinds(cfg, t, h)
        # oracle: FP32 warm-up of this head from zero, then pack
        e = np.zeros((D, D), np.uint32)
        r = np.zeros(D, np.float32)
        c = np.ones(D, np.float32)
        for (q, k, v, beta, a) in warm_inputs[(b, h)]:
            e, r, c, _, _ = orc.head_step(k32, e, r, c, np.ones(D, np.float32), q, k, v, beta, a)
        S0 = e.view(np.float32)
        e0, r0, c0, _ = orc.requant(kinds, S0, t["omega"][h], scale_mode=cfg.scale_mode)
        blk0 = orc.encode_block(kinds, cfg.unit, cfg.scale_mode, e0, r0, c0)
        assert np.array_equal(before[(b, h)], blk0), f"packed warm state differs at request {b} head {h}"
        # oracle: the timed decode step
        q, k, v, beta, a = host_slice(ins, b, h)
        e1, r1, c1, o_ref, S_pre = orc.head_step(kinds, e0, r0, c0, t["omega"][h], q, k, v, beta, a,
                                                 scale_mode=cfg.scale_mode)
        blk1 = orc.encode_block(kinds, cfg.unit, cfg.scale_mode, e1, r1, c1)
        got = dev_block(pool, t["slots"][b], h)
        if not np.array_equal(got, blk1):
            P = orc.Pool(1, 1, kinds[:1] if cfg.unit == 0 else kinds, t["omega"][h:h + 1], unit=cfg.unit,
                         scale_mode=cfg.scale_mode)
            nd, nex, other = parity._tie_analysis(orc, P, 0, S_pre, blk1, got)
            assert not other and nd == nex and nex <= parity.MAX_EXCUSED_FRACTION * D * D, \
                f"request {b} head {h}: {nd} codes differ ({nex} at ties), other bytes differ: {other}"
        od = o[b, h].cpu().numpy()
        assert parity.rel_l2(od, o_ref) <= parity.O_REL_L2, f"readout of request {b} head {h}"


class _RequestSlots:
    """The device pool seen through a request -> slot map, so that oracle slot
    i (request i of a sub-batch) compares against the device slot holding it."""

    def __init__(self, pool, dev_slots):
        self.pool, self.dev_slots = pool, [int(x) for x in dev_slots]

    def qdr_read_raw(self, i):
        return self.pool.qdr_read_raw(self.dev_slots[int(i)])

    def qdr_write_raw(self, i, raw):
        self.pool.qdr_write_raw(self.dev_slots[int(i)], raw)


def _host_rows(inputs, req):
    return tuple(np.ascontiguousarray(x[req].cpu().numpy()) for x in inputs)


def _config4_checked_pool(torch, orc, req, scale_bits=32):
    """The benchmark pool with random device-packed states in every slot and,
    in the slots of the checked requests, one host-generated dense state that
    both sides pack (so the oracle never takes a device byte).  Returns the
    config, its tables, the pool, the device slot map, the oracle pool of the
    checked requests and the device pool seen through their slots."""
    cfg = synth.CONFIGS[4]
    t = synth.static_tables(cfg)
    n = req.size
    pool = workload.make_pool(cfg, t, scale_bits=scale_bits)
    slots = torch.from_numpy(t["slots"]).cuda()
    # the other requests: random dense states generated and packed on the device
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    chunk = 32
    for s0 in range(0, cfg.B, chunk):
        S = torch.randn((chunk, cfg.H, D, D), generator=gen, device="cuda")
        S *= torch.exp(torch.randn((chunk, cfg.H, D, 1), generator=gen, device="cuda"))
        pool.qdr_pack(slots[s0:s0 + chunk].contiguous(), S)
        del S
    # the checked requests: one host-generated dense state, packed by both sides
    ref = orc.Pool(n, cfg.H, t["kinds"], t["omega"], unit=cfg.unit, gate=cfg.gate,
                   scale_mode=cfg.scale_mode, fit_iters=cfg.fit_iters, scale_bits=scale_bits).alloc()
    for i, r in enumerate(req):
        S = synth.random_state(40000 + int(r), 1, cfg.H)
        pool.qdr_pack(slots[r:r + 1].contiguous(), torch.from_numpy(S).cuda())
        ref.pack(np.array([i], np.int32), S, threads=16)
        del S
    torch.cuda.synchronize()
    view = _RequestSlots(pool, t["slots"][req])
    for i in range(n):
        assert np.array_equal(view.qdr_read_raw(i), ref.mem[i * ref.slot_stride:(i + 1) * ref.slot_stride]), \
            f"packed state of request {req[i]} differs"
    print(f"config 4 (scale bits {scale_bits}): packed states of requests {req.tolist()} match "
          f"({n} x {cfg.H} heads)", flush=True)
    return cfg, t, pool, slots, ref, view


def test_config4_every_head_of_eight_requests(torch_dev, orc):
    torch = torch_dev
    req = np.array([0, 73, 146, 219, 292, 365, 438, 511])
    n = req.size
    cfg, t, pool, slots, ref, view = _config4_checked_pool(torch, orc, req)
    ins = workload.step_inputs(cfg, t, 0)
    o = torch.empty((cfg.B, cfg.H, D), dtype=torch.float32, device="cuda")
    pool.qdr_decode_step(slots, *ins, o)
    sub = _host_rows(ins, req)
    prev = ref.mem.copy()
    rslots = np.arange(n, dtype=np.int32)
    o_ref, bad = ref.step(rslots, *sub, threads=16)
    torch.cuda.synchronize()
    assert bad == 0 and pool.qdr_poll_device_error() == 0
    rep = parity.StepReport()
    parity.compare_o(o.cpu().numpy()[req], o_ref, rep, ref.last_o_mag)
    parity.compare_pool(orc, ref, view, rslots, parity.step_state_fn(orc, ref, prev, rslots, sub), rep)
    parity.assert_step_ok(rep, "config 4 decode step")
    print(f"config 4: every head of {n} requests matches after the step: o rel L2 {rep.o_rel_l2:.2e}, "
          f"worst head {rep.o_worst_head:.2e}, excused codes {rep.codes_excused}", flush=True)
    pool.close()


# The step variants the benchmark line times on the same pool: bfloat16 scale
# factors, bfloat16 q/k/v/o, and the two-launch (readout, then write-back)
# step.  Every head of three requests against the oracle, at full size.
@pytest.mark.parametrize("variant", ["bf16_scales", "bf16_io", "split"])
def test_config4_step_variants_every_head(torch_dev, orc, variant):
    torch = torch_dev
    req = np.array([0, 255, 511])
    n = req.size
    cfg, t, pool, slots, ref, view = _config4_checked_pool(
        torch, orc, req, scale_bits=16 if variant == "bf16_scales" else 32)
    q, k, v, beta, gate = workload.step_inputs(cfg, t, 0)
    o = torch.empty((cfg.B, cfg.H, D), dtype=torch.float32, device="cuda")
    if variant == "bf16_io":
        q16, k16, v16 = (x.to(torch.bfloat16) for x in (q, k, v))
        o16 = torch.empty((cfg.B, cfg.H, D), dtype=torch.bfloat16, device="cuda")
        pool.qdr_decode_step_bf16(slots, q16, k16, v16, beta, gate, o16)
        q, k, v = (x.float() for x in (q16, k16, v16))      # the widened inputs, exact
    elif variant == "split":
        s_read, s_wb = torch.cuda.Stream(), torch.cuda.Stream()
        s_read.wait_stream(torch.cuda.current_stream())
        s_wb.wait_stream(torch.cuda.current_stream())
        pool.qdr_decode_step_split(slots, q, k, v, beta, gate, o, stream_readout=s_read, stream_writeback=s_wb)
    else:
        pool.qdr_decode_step(slots, q, k, v, beta, gate, o)
    torch.cuda.synchronize()
    assert pool.qdr_poll_device_error() == 0
    sub = _host_rows((q, k, v, beta, gate), req)
    prev = ref.mem.copy()
    rslots = np.arange(n, dtype=np.int32)
    o_ref, bad = ref.step(rslots, *sub, threads=16)
    assert bad == 0
    rep = parity.StepReport()
    if variant == "bf16_io":
        # o is the readout rounded to bfloat16: within half a bfloat16 step
        # (at most 2^-8 of the value: 8 significant bits) of the oracle's,
        # plus the readout's own bound
        o_dev = o16.float().cpu().numpy()[req].reshape(-1, D).astype(np.float64)
        o_r = np.asarray(o_ref, np.float64).reshape(-1, D)
        mag = np.asarray(ref.last_o_mag, np.float64).reshape(-1, D)
        err = np.abs(o_dev - o_r)
        bound = 2.0 ** -8 * np.abs(o_r) + parity.O_WORST_HEAD * (
            np.linalg.norm(o_r, axis=1, keepdims=True) + parity.MAG_WEIGHT * np.linalg.norm(mag, axis=1, keepdims=True))
        assert np.all(err <= bound), f"bf16 readout: worst excess {np.max(err - bound):.3e}"
        print(f"config 4 bf16_io: readout within {np.max(err / bound):.2f} of its bound", flush=True)
    else:
        parity.compare_o(o.cpu().numpy()[req], o_ref, rep, ref.last_o_mag)
    parity.compare_pool(orc, ref, view, rslots, parity.step_state_fn(orc, ref, prev, rslots, sub), rep)
    parity.assert_step_ok(rep, f"config 4 {variant} step")
    print(f"config 4 {variant}: every head of {n} requests matches after the step "
          f"(excused codes {rep.codes_excused})", flush=True)
    pool.close()


# Config 5 runs its least-squares refit; the clip-free column factor (the
# row kernel's other instantiation) is checked on one request as well.
@pytest.mark.parametrize("request_index,fit_iters", [(0, None), (170, None), (341, None), (511, None), (511, 0)])
def test_config5_every_head_of_a_request(torch_dev, orc, request_index, fit_iters):
    import dataclasses
    torch = torch_dev
    cfg = synth.CONFIGS[5]
    if fit_iters is not None:
        cfg = dataclasses.replace(cfg, fit_iters=fit_iters)
    t = synth.static_tables(cfg)
    r = int(request_index)
    pool = workload.make_pool(cfg, t)
    slots = torch.from_numpy(t["slots"]).cuda()
    pool.qdr_slot_reset(slots)
    ref = orc.Pool(1, cfg.H, t["kinds"], t["omega"], unit=cfg.unit, gate=cfg.gate,
                   scale_mode=cfg.scale_mode, fit_iters=cfg.fit_iters).alloc()
    ref.pack(np.array([0], np.int32), np.zeros((1, cfg.H, D, D), np.float32))
    view = _RequestSlots(pool, [t["slots"][r]])
    o = torch.empty((cfg.B, cfg.H, D), dtype=torch.float32, device="cuda")
    worst = worst_head = 0.0
    excused = 0
    rs = np.zeros(1, np.int32)
    for s in range(cfg.steps):
        ins = workload.step_inputs(cfg, t, s)
        pool.qdr_decode_step(slots, *ins, o)
        sub = _host_rows(ins, [r])
        prev = ref.mem.copy()
        o_ref, bad = ref.step(rs, *sub, threads=16)
        assert bad == 0
        rep = parity.StepReport()
        parity.compare_o(o[r:r + 1].cpu().numpy(), o_ref, rep, ref.last_o_mag)
        parity.compare_pool(orc, ref, view, rs, parity.step_state_fn(orc, ref, prev, rs, sub), rep)
        parity.assert_step_ok(rep, f"config 5 request {r} step {s}")
        worst, worst_head = max(worst, rep.o_rel_l2), max(worst_head, rep.o_worst_head)
        excused += rep.codes_excused
        if s % 16 == 15:
            print(f"config 5 request {r} (slot {t['slots'][r]}): {s + 1} steps match", flush=True)
    assert pool.qdr_poll_device_error() == 0
    print(f"config 5 request {r} (fit {cfg.fit_iters}): {cfg.steps} steps x {cfg.H} heads: worst o rel L2 {worst:.2e}, "
          f"worst head {worst_head:.2e}, excused codes {excused}", flush=True)
    # slots outside the slot map were never touched (zero-filled at creation)
    unmapped = sorted(set(range(cfg.num_slots)) - set(t["slots"].tolist()))
    for sl in (unmapped[0], unmapped[len(unmapped) // 2], unmapped[-1]):
        assert not pool.qdr_read_raw(sl).any(), f"unmapped slot {sl} was written"
    pool.close()
