"""Byte layout of the oracle's pool blocks, checked with an independent packer.

The reference packer below builds each column's code stream as one Python
integer (bit p of the stream = bit p of the integer) and scatters its bytes
into granules; it shares nothing with the oracle's C bit loop.
"""
import numpy as np
import pytest

from quantized_delta_rule_decode_amd import synth

D = 128


def ref_pack(kinds, unit, scale_mode, codes, fp_bits, r, c, scale_bits=32):
    G = 16 if unit == 0 else 4
    fb = 2 if scale_bits == 16 else 4          # bytes per stored factor
    widths = [int(k) for k in kinds]
    gbits = 8 * G
    ng0 = (sum(widths[:64]) + gbits - 1) // gbits
    ng1 = (sum(widths[64:]) + gbits - 1) // gbits
    ng = ng0 + ng1
    code_bytes = ng * D * G
    has_int = any(w <= 8 for w in widths)
    sbytes = (2 * D * fb if scale_mode == 0 else D * fb) if has_int else 0
    size = (code_bytes + sbytes + 255) // 256 * 256
    out = bytearray(size)
    for j in range(D):
        halves = []
        for lo in (0, 64):
            stream = 0
            pos = 0
            for i in range(lo, lo + 64):
                w = widths[i]
                if w <= 8:
                    field = int(codes[i, j]) % (1 << w)     # b-bit two's complement
                else:
                    field = int(fp_bits[i, j])
                assert 0 <= field < (1 << w)
                stream |= field << pos
                pos += w
            halves.append(stream)
        raw = halves[0].to_bytes(ng0 * G, "little") + halves[1].to_bytes(ng1 * G, "little")
        for n, byte in enumerate(raw):
            out[((n // G) * D + j) * G + n % G] = byte
    def factor_bytes(x):
        u = np.asarray(x, np.float32).view(np.uint32)
        if fb == 4:
            return u.tobytes()
        assert np.all(u & 0xFFFF == 0), "a 16-bit factor must be a bfloat16 value"
        return b"".join(int(w >> 16).to_bytes(2, "little") for w in u)

    if has_int:
        out[code_bytes:code_bytes + D * fb] = factor_bytes(r)            # r right after the codes
        if scale_mode == 0:
            out[code_bytes + D * fb:code_bytes + 2 * D * fb] = factor_bytes(c)   # then c
    return np.frombuffer(bytes(out), np.uint8)


def random_head(g, kinds):
    codes = np.zeros((D, D), np.int64)
    fp_bits = np.zeros((D, D), np.int64)
    e = np.zeros((D, D), np.uint32)
    for i, w in enumerate(kinds):
        if w <= 8:
            q = 2 ** (int(w) - 1) - 1
            codes[i] = g.integers(-q, q + 1, D)
            e[i] = codes[i].astype(np.int32).view(np.uint32)
        elif w == 16:
            fp_bits[i] = g.integers(0, 1 << 16, D)
            e[i] = fp_bits[i].astype(np.uint32)
        else:
            fp_bits[i] = g.integers(0, 1 << 32, D, dtype=np.uint64)
            e[i] = fp_bits[i].astype(np.uint32)
    r = g.lognormal(0, 1, D).astype(np.float32)
    c = g.lognormal(0, 1, D).astype(np.float32)
    return codes, fp_bits, e, r, c


KIND_SETS = {
    "int2": [2] * D, "int4": [4] * D, "int6": [6] * D, "int8": [8] * D,
    "fp16": [16] * D, "fp32": [32] * D,
    "mixed": [2, 4, 6, 8, 16, 6, 4, 2] * 16,
    "mixed_fp32": [32, 2, 2, 6] * 32,
    "odd": [6] * 127 + [2],
    "odd_halves": [6] * 63 + [2] + [16] * 3 + [6] * 61,
}


# whole-head units have one kind per head, so mixed kind sets go with row units only
LAYOUT_CASES = [(name, unit) for name in sorted(KIND_SETS) for unit in (0, 1)
                if unit == 1 or len(set(KIND_SETS[name])) == 1]


@pytest.mark.parametrize("name,unit", LAYOUT_CASES)
@pytest.mark.parametrize("scale_mode", [0, 1])
@pytest.mark.parametrize("sb", [32, 16])
def test_encode_matches_reference_packer(orc, name, unit, scale_mode, sb):
    kinds = np.array(KIND_SETS[name], np.uint8)
    g = np.random.default_rng(hash((name, unit, scale_mode, sb)) % 2 ** 32)
    codes, fp_bits, e, r, c = random_head(g, kinds)
    if sb == 16:
        # bfloat16 factors: distinct random values whose low 16 bits are zero
        r = (r.view(np.uint32) & 0xFFFF0000).view(np.float32)
        c = (c.view(np.uint32) & 0xFFFF0000).view(np.float32)
    if not any(k <= 8 for k in kinds):
        r = np.zeros(D, np.float32)
    blob = orc.encode_block(kinds, unit, scale_mode, e, r, c, scale_bits=sb)
    ref = ref_pack(kinds, unit, scale_mode, codes, fp_bits, r, c, scale_bits=sb)
    assert blob.size == ref.size == orc.block_bytes(kinds, unit, scale_mode, sb)
    assert np.array_equal(blob, ref)
    e2, r2, c2 = orc.decode_block(kinds, unit, scale_mode, blob, scale_bits=sb)
    assert np.array_equal(e2, e)
    if any(k <= 8 for k in kinds):
        assert np.array_equal(r2, r)
        if scale_mode == 0:
            assert np.array_equal(c2, c)
        else:
            assert np.all(c2 == 1.0)


def test_block_sizes(orc):
    # whole-head units: codes are d*d*b/8 bytes; scales 1 KiB (dual) / 512 B (row absmax)
    for b in (2, 4, 6, 8):
        k = np.full(D, b, np.uint8)
        assert orc.code_bytes(k, 0) == D * D * b // 8
        assert orc.block_bytes(k, 0, 0) == D * D * b // 8 + 1024
        assert orc.block_bytes(k, 0, 1) == D * D * b // 8 + 512
    assert orc.block_bytes(np.full(D, 16, np.uint8), 0, 0) == 32768
    # an FP32 head is the uncompressed 128 x 128 fp32 state: 64 KiB
    assert orc.block_bytes(np.full(D, 32, np.uint8), 0, 0) == 65536
    # row units pad each half of a column stream to whole 32-bit words
    k = np.array([6] * 127 + [2], np.uint8)     # 384 + 380 bits -> 12 + 12 words
    assert orc.code_bytes(k, 1) == 24 * 4 * D
    k = np.array([6] * 63 + [2] + [4] * 64, np.uint8)   # 380 -> 12 words, 256 -> 8 words
    assert orc.code_bytes(k, 1) == 20 * 4 * D


def test_pages_state_bytes(orc):
    """Uncompressed state of one slot of the 2304-head GDN model (printed figures)."""
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
    heads = gold["qwen_recurrent_heads"]["value"]
    dk, dv = gold["state_shape"]["value"]
    P = orc.Pool(1, heads, np.full(heads, 32, np.uint8), np.ones((heads, D), np.float32))
    # an all-FP32 slot is exactly heads x d_k x d_v fp32 values: 144 MiB, which sits
    # inside the printed 146.8125 MiB per slot (the remainder is non-recurrent state)
    assert P.slot_stride == heads * dk * dv * 4 == 144 * 2 ** 20
    assert 0 < gold["fp32_slot_mib"]["value"] - P.slot_stride / 2 ** 20 < 0.02 * 146.8125
    # the printed compression is 32 / (bits per value)
    for row in gold["compression"]:
        assert abs(32.0 / row["bits_per_value"] - row["ratio"]) <= 0.005
    # the synthetic allocations reach the printed actual mean widths
    t4 = synth.static_tables(synth.CONFIGS[4])
    t3 = synth.static_tables(synth.CONFIGS[3])
    assert abs(t4["kinds"].mean() - gold["actual_mean_bits"]["nominal6"]) < 0.005
    assert abs(t3["kinds"].mean() - gold["actual_mean_bits"]["nominal4"]) < 0.005


def test_pool_layout_and_slots(orc):
    cfg = synth.CONFIGS[3]
    t = synth.static_tables(cfg)
    H = 6
    kinds = t["kinds"][: H * D]
    P = orc.Pool(5, H, kinds, t["omega"][:H], unit=1, gate=1)
    sizes = [P.block_size(h) for h in range(H)]
    assert P.head_off.tolist() == list(np.cumsum([0] + sizes[:-1]))
    assert P.slot_stride == sum(sizes) and P.total == 5 * sum(sizes)
    assert all(s % 256 == 0 for s in sizes)


def test_pool_step_composes_head_steps(orc):
    """Pool step = decode block, head step, encode block, for every mapped slot."""
    cfg = synth.CONFIGS[2]
    t = synth.static_tables(cfg)
    H = 5
    kinds = np.array([16, 8, 6, 4, 6], np.uint8)
    P = orc.Pool(4, H, kinds, t["omega"][:H], unit=0, gate=0).alloc()
    S0 = synth.random_state(3, 4, H)
    P.pack(np.arange(4), S0)
    before = P.mem.copy()
    slots = np.array([2, -1, 0], np.int32)
    g = np.random.default_rng(0)
    q = g.standard_normal((3, H, D)).astype(np.float32)
    k = g.standard_normal((3, H, D)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal((3, H, D)).astype(np.float32)
    beta = g.uniform(size=(3, H)).astype(np.float32)
    gate = g.uniform(0.5, 1, size=(3, H)).astype(np.float32)
    o, bad = P.step(slots, q, k, v, beta, gate, threads=3)
    assert bad == 0
    assert np.all(o[1] == 0)
    for b, slot in enumerate(slots):
        if slot < 0:
            continue
        for h in range(H):
            hk = P.head_kinds(h)
            off = slot * P.slot_stride + int(P.head_off[h])
            blk = before[off: off + P.block_size(h)]
            e, r, c = orc.decode_block(hk, 0, 0, blk)
            e2, r2, c2, o_ref, _ = orc.head_step(hk, e, r, c, t["omega"][h], q[b, h], k[b, h],
                                                 v[b, h], float(beta[b, h]),
                                                 np.full(D, gate[b, h], np.float32))
            assert np.array_equal(o[b, h], o_ref)
            assert np.array_equal(P.block_view(slot, h), orc.encode_block(hk, 0, 0, e2, r2, c2))
    # slot 1 and 3 untouched, slot 3 never listed
    for s in (1, 3):
        a, b_ = s * P.slot_stride, (s + 1) * P.slot_stride
        assert np.array_equal(P.mem[a:b_], before[a:b_])
    # out-of-range slots are reported and give zero output
    o, bad = P.step(np.array([7, 0], np.int32), q[:2], k[:2], v[:2], beta[:2], gate[:2])
    assert bad == 1 and np.all(o[0] == 0)


def test_unpack_pack_roundtrip(orc):
    H = 3
    kinds = np.array([8, 6, 32], np.uint8)
    P = orc.Pool(2, H, kinds, np.ones((H, D), np.float32)).alloc()
    S = synth.random_state(9, 2, H)
    P.pack(np.arange(2), S)
    X = P.unpack(np.arange(2))
    assert np.array_equal(X[:, 2], S[:, 2])
    # the FP32 head is stored verbatim: re-packing the restored state gives the same bytes
    mem = P.mem.copy()
    P.pack(np.arange(2), X)
    for slot in range(2):
        assert np.array_equal(P.block_view(slot, 2), mem[slot * P.slot_stride + int(P.head_off[2]):][:P.block_size(2)])
