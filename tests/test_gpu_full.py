"""Full-size device runs, checked on sampled (request, head) pairs.

Config 4 is the benchmark's own launch: the 512 x 2304-head GDN pool, warm
state from 256 FP32 decode steps, then one quantised decode step.  Config 5
is the (5B+1)-slot KDA pool with a random slot map, 64 decode steps from the
zero state.  The oracle recomputes each sampled head on its own from the same
seeded inputs (copied from the device generator) and never reads a byte the
device produced; unmapped slots are checked to stay untouched.
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


def test_config5_slot_pool_sampled(torch_dev, orc):
    torch = torch_dev
    cfg = synth.CONFIGS[5]
    t = synth.static_tables(cfg)
    # per-head mean width as the "kind" used to spread the samples
    hk = t["kinds"].reshape(cfg.H, D)
    bucket = np.digitize(hk.mean(axis=1), [4.0, 4.3, 4.6])
    samples = pick_samples(bucket, cfg.B, cfg.H, per_kind=2, seed=1)
    pool = workload.make_pool(cfg, t)
    slots = torch.from_numpy(t["slots"]).cuda()
    pool.qdr_slot_reset(slots)
    o = torch.empty((cfg.B, cfg.H, D), dtype=torch.float32, device="cuda")
    state = {}
    for (b, h) in samples:
        kinds = head_kinds(cfg, t, h)
        e, r, c, _ = orc.requant(kinds, np.zeros((D, D), np.float32), t["omega"][h])
        state[(b, h)] = (e, r, c)
    worst = 0.0
    steps = cfg.steps
    for s in range(steps):
        ins = workload.step_inputs(cfg, t, s)
        pool.qdr_decode_step(slots, *ins, o)
        for (b, h) in samples:
            kinds = head_kinds(cfg, t, h)
            q, k, v, beta, a = host_slice(ins, b, h)
            e, r, c = state[(b, h)]
            e, r, c, o_ref, _ = orc.head_step(kinds, e, r, c, t["omega"][h], q, k, v, beta, a)
            state[(b, h)] = (e, r, c)
            worst = max(worst, parity.rel_l2(o[b, h].cpu().numpy(), o_ref))
    torch.cuda.synchronize()
    assert pool.qdr_poll_device_error() == 0
    assert worst <= parity.O_REL_L2
    for (b, h) in samples:
        kinds = head_kinds(cfg, t, h)
        e, r, c = state[(b, h)]
        want = orc.encode_block(kinds, cfg.unit, cfg.scale_mode, e, r, c)
        got = dev_block(pool, t["slots"][b], h)
        assert np.array_equal(got, want), f"request {b} (slot {t['slots'][b]}) head {h} differs"
    # slots outside the slot map were never touched (zero-filled at creation)
    unmapped = sorted(set(range(cfg.num_slots)) - set(t["slots"].tolist()))
    for sl in (unmapped[0], unmapped[len(unmapped) // 2], unmapped[-1]):
        assert not pool.qdr_read_raw(sl).any(), f"unmapped slot {sl} was written"
