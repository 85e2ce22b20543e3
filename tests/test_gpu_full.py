"""Full-size device runs in the benchmark's launch configuration.

Config 4 is the benchmark's own launch: the 512 x 2304-head GDN pool, one
quantised decode step over every request.  Two checks: every head of eight
requests (0 and 511 among them) from a dense state generated on the host,
which both sides pack; and sampled heads of the benchmark's own warm state
(256 FP32 decode steps, then pack).  Config 5 is the (5B+1)-slot KDA pool
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


def test_config4_every_head_of_eight_requests(torch_dev, orc):
    torch = torch_dev
    cfg = synth.CONFIGS[4]
    t = synth.static_tables(cfg)
    req = np.array([0, 73, 146, 219, 292, 365, 438, 511])
    n = req.size
    pool = workload.make_pool(cfg, t)
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
                   scale_mode=cfg.scale_mode, fit_iters=cfg.fit_iters).alloc()
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
    print(f"config 4: packed states of requests {req.tolist()} match ({n} x {cfg.H} heads)", flush=True)
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


@pytest.mark.parametrize("request_index", [0, 170, 341, 511])
def test_config5_every_head_of_a_request(torch_dev, orc, request_index):
    torch = torch_dev
    cfg = synth.CONFIGS[5]
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
    print(f"config 5 request {r}: {cfg.steps} steps x {cfg.H} heads: worst o rel L2 {worst:.2e}, "
          f"worst head {worst_head:.2e}, excused codes {excused}", flush=True)
    # slots outside the slot map were never touched (zero-filled at creation)
    unmapped = sorted(set(range(cfg.num_slots)) - set(t["slots"].tolist()))
    for sl in (unmapped[0], unmapped[len(unmapped) // 2], unmapped[-1]):
        assert not pool.qdr_read_raw(sl).any(), f"unmapped slot {sl} was written"
    pool.close()
