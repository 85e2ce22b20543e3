"""ctypes front end of the CPU oracle (``qdr_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library.  Arrays are numpy,
C-contiguous; nothing here performs any of the method's arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qdr_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# an alternate build of the same source (e.g. a sanitizer build) may be named here
LIB_OVERRIDE = os.environ.get("QDR_ORACLE_LIB")

INT2, INT4, INT6, INT8, FP16, FP32 = 2, 4, 6, 8, 16, 32
UNIT_HEAD, UNIT_ROW = 0, 1
SCALE_DUAL, SCALE_ROW_ABSMAX = 0, 1
GATE_SCALAR, GATE_DIAG = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no contraction, IEEE fp32)."""
    if force or not os.path.exists(LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-pthread", SRC, "-o", LIB + ".tmp", "-lm"]
        subprocess.check_call(cmd)
        os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if LIB_OVERRIDE:
            _lib = ctypes.CDLL(os.path.abspath(LIB_OVERRIDE))
        else:
            if not os.path.exists(LIB):
                build()
            _lib = ctypes.CDLL(LIB)
        _declare(_lib)
    return _lib


_p = ctypes.c_void_p


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_slots", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("unit", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("scale_mode", ctypes.c_int32), ("fit_iters", ctypes.c_int32),
                ("kinds", _p), ("omega", _p), ("scale_bits", ctypes.c_int32)]


def _declare(L):
    L.or_f32_to_f16.restype = ctypes.c_uint16
    L.or_f32_to_f16.argtypes = [ctypes.c_float]
    L.or_f16_to_f32.restype = ctypes.c_float
    L.or_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.or_fold_sum.restype = ctypes.c_float
    L.or_fold_sum.argtypes = [_p, ctypes.c_int]
    L.or_dequant.argtypes = [ctypes.c_int, _p, _p, _p, _p, _p, _p]
    L.or_delta_update.argtypes = [ctypes.c_int, _p, _p, _p, ctypes.c_float, _p, _p]
    L.or_readout.argtypes = [ctypes.c_int, _p, _p, _p]
    L.or_requant.argtypes = [ctypes.c_int, _p, _p, _p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             _p, _p, _p, _p]
    L.or_head_step.argtypes = [ctypes.c_int, _p, _p, _p, _p, _p, ctypes.c_int,
                               ctypes.c_int, ctypes.c_int, _p, _p, _p, ctypes.c_float, _p, _p, _p]
    L.or_bf16_up.restype = ctypes.c_float
    L.or_bf16_up.argtypes = [ctypes.c_float]
    L.or_bf16_nearest.restype = ctypes.c_float
    L.or_bf16_nearest.argtypes = [ctypes.c_float]
    L.or_block_bytes.restype = ctypes.c_size_t
    L.or_block_bytes.argtypes = [_p, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.or_code_bytes.restype = ctypes.c_size_t
    L.or_code_bytes.argtypes = [_p, ctypes.c_int]
    L.or_encode_block.argtypes = [_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _p, _p, _p, _p]
    L.or_decode_block.argtypes = [_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _p, _p, _p, _p]
    L.or_pool_layout.argtypes = [ctypes.POINTER(PoolDesc), _p, _p, _p]
    L.or_pool_step.restype = ctypes.c_int
    L.or_pool_step.argtypes = [ctypes.POINTER(PoolDesc), _p, _p, ctypes.c_int32,
                               _p, _p, _p, _p, _p, _p, ctypes.c_int, _p]
    L.or_readout_magnitude.argtypes = [ctypes.c_int, _p, _p, _p]
    L.or_pool_pack.restype = ctypes.c_int
    L.or_pool_pack.argtypes = [ctypes.POINTER(PoolDesc), _p, _p, ctypes.c_int32, _p,
                               ctypes.c_int]
    L.or_pool_unpack.restype = ctypes.c_int
    L.or_pool_unpack.argtypes = [ctypes.POINTER(PoolDesc), _p, _p, ctypes.c_int32, _p,
                                 ctypes.c_int]


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- scalars
def f32_to_f16(x: float) -> int:
    return int(lib().or_f32_to_f16(ctypes.c_float(x)))


def f16_to_f32(h: int) -> float:
    return float(lib().or_f16_to_f32(ctypes.c_uint16(h)))


def bf16_up(x: float) -> float:
    return float(lib().or_bf16_up(ctypes.c_float(x)))


def bf16_nearest(x: float) -> float:
    return float(lib().or_bf16_nearest(ctypes.c_float(x)))


def fold_sum(x) -> float:
    x = _c(x, np.float32).copy()
    return float(lib().or_fold_sum(_ptr(x), x.size))


# ---------------------------------------------------------------- dense head
def dequant(kinds, e, r, c, a):
    kinds = _c(kinds, np.uint8)
    d = kinds.size
    e = _c(e, np.uint32)
    r, c, a = _c(r, np.float32), _c(c, np.float32), _c(a, np.float32)
    Sp = np.empty((d, d), np.float32)
    lib().or_dequant(d, _ptr(kinds), _ptr(e), _ptr(r), _ptr(c), _ptr(a), _ptr(Sp))
    return Sp


def delta_update(Sp, k, v, beta):
    Sp = _c(Sp, np.float32)
    d = Sp.shape[0]
    k, v = _c(k, np.float32), _c(v, np.float32)
    S = np.empty((d, d), np.float32)
    u = np.empty(d, np.float32)
    lib().or_delta_update(d, _ptr(Sp), _ptr(k), _ptr(v), ctypes.c_float(beta), _ptr(S), _ptr(u))
    return S, u


def readout_magnitude(S, q):
    S = _c(S, np.float32)
    d = S.shape[0]
    q = _c(q, np.float32)
    m = np.empty(d, np.float32)
    lib().or_readout_magnitude(d, _ptr(S), _ptr(q), _ptr(m))
    return m


def readout(S, q):
    S = _c(S, np.float32)
    d = S.shape[0]
    q = _c(q, np.float32)
    o = np.empty(d, np.float32)
    lib().or_readout(d, _ptr(S), _ptr(q), _ptr(o))
    return o


def requant(kinds, S, omega, scale_mode=SCALE_DUAL, fit_iters=0, scale_bits=32):
    kinds = _c(kinds, np.uint8)
    d = kinds.size
    S = _c(S, np.float32)
    omega = _c(omega, np.float32)
    e = np.zeros((d, d), np.uint32)
    r = np.empty(d, np.float32)
    c = np.empty(d, np.float32)
    m = np.empty(d, np.float32)
    lib().or_requant(d, _ptr(kinds), _ptr(S), _ptr(omega), scale_mode, fit_iters, scale_bits,
                     _ptr(e), _ptr(r), _ptr(c), _ptr(m))
    return e, r, c, m


def head_step(kinds, e, r, c, omega, q, k, v, beta, a, scale_mode=SCALE_DUAL, fit_iters=0, scale_bits=32):
    """Returns (e', r', c', o, S_pre) without modifying the inputs."""
    kinds = _c(kinds, np.uint8)
    d = kinds.size
    e = _c(e, np.uint32).copy()
    r = _c(r, np.float32).copy()
    c = _c(c, np.float32).copy()
    omega, q, k, v, a = (_c(x, np.float32) for x in (omega, q, k, v, a))
    o = np.empty(d, np.float32)
    S_pre = np.empty((d, d), np.float32)
    lib().or_head_step(d, _ptr(kinds), _ptr(e), _ptr(r), _ptr(c), _ptr(omega), scale_mode,
                       fit_iters, scale_bits, _ptr(q), _ptr(k), _ptr(v), ctypes.c_float(beta), _ptr(a),
                       _ptr(o), _ptr(S_pre))
    return e, r, c, o, S_pre


def codes_signed(e, kinds):
    """View of the integer codes of INT rows as int32 (other rows untouched)."""
    return np.asarray(e).view(np.int32)


# ---------------------------------------------------------------- blocks
def block_bytes(kinds, unit, scale_mode, scale_bits=32):
    kinds = _c(kinds, np.uint8)
    return int(lib().or_block_bytes(_ptr(kinds), unit, scale_mode, scale_bits))


def code_bytes(kinds, unit):
    kinds = _c(kinds, np.uint8)
    return int(lib().or_code_bytes(_ptr(kinds), unit))


def encode_block(kinds, unit, scale_mode, e, r, c, scale_bits=32):
    kinds = _c(kinds, np.uint8)
    e, r, c = _c(e, np.uint32), _c(r, np.float32), _c(c, np.float32)
    out = np.zeros(block_bytes(kinds, unit, scale_mode, scale_bits), np.uint8)
    lib().or_encode_block(_ptr(kinds), unit, scale_mode, scale_bits, _ptr(e), _ptr(r), _ptr(c), _ptr(out))
    return out


def decode_block(kinds, unit, scale_mode, block, scale_bits=32):
    kinds = _c(kinds, np.uint8)
    block = _c(block, np.uint8)
    e = np.zeros((128, 128), np.uint32)
    r = np.empty(128, np.float32)
    c = np.empty(128, np.float32)
    lib().or_decode_block(_ptr(kinds), unit, scale_mode, scale_bits, _ptr(block), _ptr(e), _ptr(r), _ptr(c))
    return e, r, c


# ---------------------------------------------------------------- pool
class Pool:
    """Host image of a state pool in the oracle's own layout."""

    def __init__(self, num_slots, num_heads, kinds, omega, unit=UNIT_HEAD,
                 gate=GATE_SCALAR, scale_mode=SCALE_DUAL, fit_iters=0, scale_bits=32):
        self.kinds = _c(kinds, np.uint8)
        self.omega = _c(omega, np.float32)
        self.scale_bits = scale_bits
        self.desc = PoolDesc(num_slots, num_heads, unit, gate, scale_mode, fit_iters,
                             _ptr(self.kinds).value, _ptr(self.omega).value, scale_bits)
        H = num_heads
        self.head_off = np.zeros(H, np.uint64)
        stride = ctypes.c_uint64(0)
        total = ctypes.c_uint64(0)
        lib().or_pool_layout(ctypes.byref(self.desc), _ptr(self.head_off),
                             ctypes.byref(stride), ctypes.byref(total))
        self.slot_stride = int(stride.value)
        self.total = int(total.value)
        self.num_slots, self.num_heads = num_slots, num_heads
        self.unit, self.gate, self.scale_mode, self.fit_iters = unit, gate, scale_mode, fit_iters
        self.mem = None

    def alloc(self):
        self.mem = np.zeros(self.total, np.uint8)
        return self

    def head_kinds(self, h):
        if self.unit == UNIT_HEAD:
            return np.full(128, self.kinds[h], np.uint8)
        return self.kinds[h * 128:(h + 1) * 128]

    def block_size(self, h):
        return block_bytes(self.head_kinds(h), self.unit, self.scale_mode, self.scale_bits)

    def block_view(self, slot, h):
        off = slot * self.slot_stride + int(self.head_off[h])
        return self.mem[off: off + self.block_size(h)]

    def step(self, slots, q, k, v, beta, gate, threads=1):
        """One decode step of the listed slots; returns (o, number of bad
        slots).  The readout magnitudes of the step are kept in last_o_mag."""
        slots = _c(slots, np.int32)
        B = slots.size
        q, k, v, beta, gate = (_c(x, np.float32) for x in (q, k, v, beta, gate))
        o = np.zeros((B, self.num_heads, 128), np.float32)
        self.last_o_mag = np.zeros((B, self.num_heads, 128), np.float32)
        bad = lib().or_pool_step(ctypes.byref(self.desc), _ptr(self.mem), _ptr(slots), B,
                                 _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(gate), _ptr(o),
                                 threads, _ptr(self.last_o_mag))
        return o, bad

    def pack(self, slots, S, threads=1):
        slots = _c(slots, np.int32)
        S = _c(S, np.float32)
        return lib().or_pool_pack(ctypes.byref(self.desc), _ptr(self.mem), _ptr(slots),
                                  slots.size, _ptr(S), threads)

    def unpack(self, slots, threads=1):
        slots = _c(slots, np.int32)
        S = np.zeros((slots.size, self.num_heads, 128, 128), np.float32)
        lib().or_pool_unpack(ctypes.byref(self.desc), _ptr(self.mem), _ptr(slots), slots.size,
                             _ptr(S), threads)
        return S
