"""The C-ABI library loads, exports every declared entry point, and its pure
host logic (descriptor checks, pool layout) agrees with the oracle's layout.
No GPU needed: nothing here enqueues device work."""
import ctypes
import os
import re

import numpy as np
import pytest

from quantized_delta_rule_decode_amd import qdr, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "qdr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qdr_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(qdr.LIB_PATH):
        from quantized_delta_rule_decode_amd import build
        build.build()
    return qdr.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 15
    assert sorted(names) == sorted(qdr.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.qdr_last_error() == b""


def _bytes(**kw):
    return qdr.qdr_pool_bytes(**kw)


@pytest.mark.parametrize("sb", [32, 16])
@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_pool_bytes_match_oracle_layout(orc, lib, cid, sb):
    cfg = synth.CONFIGS[cid]
    t = synth.static_tables(cfg)
    n = _bytes(num_slots=cfg.num_slots, num_heads=cfg.H, kinds=t["kinds"], omega=t["omega"],
               unit=cfg.unit, gate=cfg.gate, scale_mode=cfg.scale_mode, scale_bits=sb)
    P = orc.Pool(cfg.num_slots, cfg.H, t["kinds"], t["omega"], unit=cfg.unit, gate=cfg.gate,
                 scale_mode=cfg.scale_mode, scale_bits=sb)
    assert n == P.total


def test_config4_pool_size():
    """The 6-bit pool of 512 requests x 2304 heads holds about 15 GB of codes."""
    cfg = synth.CONFIGS[4]
    t = synth.static_tables(cfg)
    n = _bytes(num_slots=cfg.num_slots, num_heads=cfg.H, kinds=t["kinds"], omega=t["omega"])
    codes = 512 * sum(128 * 128 * int(k) // 8 for k in t["kinds"])
    assert 15.0e9 < codes < 15.5e9
    assert codes < n < codes * 1.1


@pytest.mark.parametrize("bad", [
    dict(num_slots=0), dict(num_heads=0), dict(unit=2), dict(gate=5), dict(scale_mode=3),
    dict(fit_iters=2), dict(fit_iters=1, scale_mode=1), dict(scale_bits=8), dict(scale_bits=-16),
    dict(kinds_value=5), dict(omega_value=0.0),
    dict(omega_value=float("nan")), dict(omega_value=2.0 ** 41), dict(omega_none=True),
])
def test_descriptor_errors(lib, bad):
    H = 3
    kw = dict(num_slots=2, num_heads=H, kinds=np.full(H, 6, np.uint8), omega=np.ones((H, 128), np.float32))
    if "kinds_value" in bad:
        kw["kinds"] = np.array([6, bad.pop("kinds_value"), 6], np.uint8)
    if "omega_value" in bad:
        om = np.ones((H, 128), np.float32)
        om[1, 7] = bad.pop("omega_value")
        kw["omega"] = om
    if bad.pop("omega_none", False):
        kw["omega"] = None
    kw.update(bad)
    with pytest.raises(qdr.QdrError) as ei:
        _bytes(**kw)
    assert ei.value.status in (-1, -5)
    assert lib.qdr_last_error() != b""


def test_row_absmax_needs_no_omega(lib):
    assert _bytes(num_slots=1, num_heads=1, kinds=[8], omega=None, scale_mode=1) == 16384 + 512
    assert _bytes(num_slots=1, num_heads=1, kinds=[8], omega=None, scale_mode=1, scale_bits=16) == 16384 + 256


def test_null_arguments_rejected(lib):
    P = ctypes.c_void_p
    assert lib.qdr_pool_bytes(None, None) == -1
    assert lib.qdr_pool_destroy(None) == 0
    assert lib.qdr_decode_step(None, None, 0, None, None, None, None, None, None, None) == -1
    assert lib.qdr_decode_step_split(None, None, 0, None, None, None, None, None, None, None, None) == -1
    assert lib.qdr_decode_step_bf16(None, None, 0, None, None, None, None, None, None, None) == -1
    assert lib.qdr_pack(None, None, 1, None, None) == -1
    flags = ctypes.c_uint32(0)
    assert lib.qdr_poll_device_error(None, ctypes.byref(flags)) == -1
    assert lib.qdr_get_layout(None, None) == -1
