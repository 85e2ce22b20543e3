"""Python binding of libqdr (include/qdr.h): argument marshalling only.

Every function here has the name of the C entry point it calls.  Tensors are
torch tensors on the current HIP device; the library receives their device
pointers and the current stream.  There is no fallback: if libqdr.so is not
built, or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqdr.so")

DIM = 128
GATE_SCALAR, GATE_DIAG = 0, 1
UNIT_HEAD, UNIT_ROW = 0, 1
SCALE_DUAL, SCALE_ROW_ABSMAX = 0, 1
K_INT2, K_INT4, K_INT6, K_INT8, K_FP16, K_FP32 = 2, 4, 6, 8, 16, 32
DEVERR_SLOT = 1

_STATUS = {0: "QDR_OK", -1: "QDR_E_INVAL", -2: "QDR_E_NOMEM", -3: "QDR_E_DEVICE",
           -4: "QDR_E_SLOT", -5: "QDR_E_UNSUPPORTED"}


class QdrError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: {_STATUS.get(status, status)}: {msg}")
        self.status = status


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_slots", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("unit", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("scale_mode", ctypes.c_int32), ("fit_iters", ctypes.c_int32),
                ("kinds", ctypes.c_void_p), ("omega", ctypes.c_void_p),
                ("scale_bits", ctypes.c_int32)]


class Layout(ctypes.Structure):
    _fields_ = [("slot_stride", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64),
                ("num_slots", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_off", ctypes.POINTER(ctypes.c_uint64)),
                ("head_bytes", ctypes.POINTER(ctypes.c_uint32)),
                ("code_bytes", ctypes.POINTER(ctypes.c_uint32)),
                ("base", ctypes.c_void_p), ("bits_per_value", ctypes.c_double)]


EXPORTS = ["qdr_pool_bytes", "qdr_pool_create", "qdr_pool_destroy", "qdr_slot_reset",
           "qdr_pack", "qdr_unpack", "qdr_decode_step", "qdr_decode_step_split", "qdr_decode_step_bf16", "qdr_get_layout", "qdr_read_raw",
           "qdr_write_raw", "qdr_poll_device_error", "qdr_last_error", "qdr_clock_probe"]

_lib = None


def load():
    """Load libqdr.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with quantized_delta_rule_decode_amd/build.py")
    # torch's HIP runtime must be the process's HIP runtime: importing torch
    # first makes libqdr.so bind to the already loaded libamdhip64.so.7
    # instead of loading a second runtime instance.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "qdr_pool_bytes": [ctypes.POINTER(PoolDesc), ctypes.POINTER(SZ)],
        "qdr_pool_create": [ctypes.POINTER(PoolDesc), P, SZ, ctypes.POINTER(P)],
        "qdr_pool_destroy": [P],
        "qdr_slot_reset": [P, P, I32, P],
        "qdr_pack": [P, P, I32, P, P],
        "qdr_unpack": [P, P, I32, P, P],
        "qdr_decode_step": [P, P, I32, P, P, P, P, P, P, P],
        "qdr_decode_step_split": [P, P, I32, P, P, P, P, P, P, P, P],
        "qdr_decode_step_bf16": [P, P, I32, P, P, P, P, P, P, P],
        "qdr_get_layout": [P, ctypes.POINTER(Layout)],
        "qdr_read_raw": [P, I32, P, SZ, P],
        "qdr_write_raw": [P, I32, P, SZ, P],
        "qdr_poll_device_error": [P, ctypes.POINTER(ctypes.c_uint32)],
        "qdr_clock_probe": [P, I32, P],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.qdr_last_error.argtypes = []
    L.qdr_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(fn, status):
    if status != 0:
        raise QdrError(fn, status, load().qdr_last_error().decode())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dptr(t, dtype, name, numel=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _desc(num_slots, num_heads, kinds, omega, unit, gate, scale_mode, fit_iters, scale_bits=32):
    kinds = np.ascontiguousarray(kinds, np.uint8)
    om = None if omega is None else np.ascontiguousarray(omega, np.float32)
    d = PoolDesc(num_slots, num_heads, DIM, DIM, unit, gate, scale_mode, fit_iters,
                 kinds.ctypes.data, None if om is None else om.ctypes.data, scale_bits)
    return d, (kinds, om)


def qdr_pool_bytes(num_slots, num_heads, kinds, omega, unit=UNIT_HEAD, gate=GATE_SCALAR,
                   scale_mode=SCALE_DUAL, fit_iters=0, scale_bits=32) -> int:
    d, keep = _desc(num_slots, num_heads, kinds, omega, unit, gate, scale_mode, fit_iters, scale_bits)
    n = ctypes.c_size_t(0)
    _check("qdr_pool_bytes", load().qdr_pool_bytes(ctypes.byref(d), ctypes.byref(n)))
    return int(n.value)


def qdr_clock_probe(out, iters, stream=None):
    """Enqueue the shader-clock probe; out: torch.int64 device tensor of >= 5
    elements (see include/qdr.h).  Returns nothing; read out after the
    stream completes: MHz = 100 * (out[2] - out[0]) / (out[3] - out[1])."""
    import torch
    if out.numel() < 5:
        raise ValueError(f"out has {out.numel()} elements, expected at least 5")
    _check("qdr_clock_probe", load().qdr_clock_probe(_dptr(out, torch.int64, "out"), int(iters), _stream(stream)))


class Pool:
    """A state pool (qdr_pool_create ... qdr_pool_destroy)."""

    def __init__(self, num_slots, num_heads, kinds, omega, unit=UNIT_HEAD, gate=GATE_SCALAR,
                 scale_mode=SCALE_DUAL, fit_iters=0, dev_mem=None, scale_bits=32):
        self.num_slots, self.num_heads = int(num_slots), int(num_heads)
        self.unit, self.gate, self.scale_mode, self.fit_iters = unit, gate, scale_mode, fit_iters
        self.scale_bits = scale_bits
        d, keep = _desc(num_slots, num_heads, kinds, omega, unit, gate, scale_mode, fit_iters, scale_bits)
        h = ctypes.c_void_p(None)
        mem_ptr, mem_bytes = None, 0
        if dev_mem is not None:
            mem_ptr, mem_bytes = ctypes.c_void_p(dev_mem.data_ptr()), dev_mem.numel() * dev_mem.element_size()
        self._dev_mem = dev_mem
        _check("qdr_pool_create", load().qdr_pool_create(ctypes.byref(d), mem_ptr, mem_bytes, ctypes.byref(h)))
        self._h = h
        lay = Layout()
        _check("qdr_get_layout", load().qdr_get_layout(self._h, ctypes.byref(lay)))
        H = self.num_heads
        self.slot_stride = int(lay.slot_stride)
        self.total_bytes = int(lay.total_bytes)
        self.head_off = np.ctypeslib.as_array(lay.head_off, shape=(H,)).copy()
        self.head_bytes = np.ctypeslib.as_array(lay.head_bytes, shape=(H,)).copy()
        self.code_bytes = np.ctypeslib.as_array(lay.code_bytes, shape=(H,)).copy()
        self.base = int(lay.base)
        self.bits_per_value = float(lay.bits_per_value)

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            _check("qdr_pool_destroy", load().qdr_pool_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # ---- entry points (same names as the C ABI)
    def qdr_slot_reset(self, slots, stream=None):
        import torch
        _check("qdr_slot_reset", load().qdr_slot_reset(
            self._h, _dptr(slots, torch.int32, "slots"), slots.numel(), _stream(stream)))

    def qdr_pack(self, slots, S, stream=None):
        import torch
        n = slots.numel()
        _check("qdr_pack", load().qdr_pack(
            self._h, _dptr(slots, torch.int32, "slots"), n,
            _dptr(S, torch.float32, "S", n * self.num_heads * DIM * DIM), _stream(stream)))

    def qdr_unpack(self, slots, S_out, stream=None):
        import torch
        n = slots.numel()
        _check("qdr_unpack", load().qdr_unpack(
            self._h, _dptr(slots, torch.int32, "slots"), n,
            _dptr(S_out, torch.float32, "S_out", n * self.num_heads * DIM * DIM), _stream(stream)))

    def qdr_decode_step(self, slots, q, k, v, beta, gate, o, stream=None):
        import torch
        B, H = slots.numel(), self.num_heads
        f32 = torch.float32
        gn = B * H if self.gate == GATE_SCALAR else B * H * DIM
        _check("qdr_decode_step", load().qdr_decode_step(
            self._h, _dptr(slots, torch.int32, "slots"), B,
            _dptr(q, f32, "q", B * H * DIM), _dptr(k, f32, "k", B * H * DIM),
            _dptr(v, f32, "v", B * H * DIM), _dptr(beta, f32, "beta", B * H),
            _dptr(gate, f32, "gate", gn), _dptr(o, f32, "o", B * H * DIM), _stream(stream)))

    def qdr_decode_step_bf16(self, slots, q, k, v, beta, gate, o, stream=None):
        """q, k, v, o: torch.bfloat16 [B][H][128]; beta, gate fp32."""
        import torch
        B, H = slots.numel(), self.num_heads
        bf, f32 = torch.bfloat16, torch.float32
        gn = B * H if self.gate == GATE_SCALAR else B * H * DIM
        _check("qdr_decode_step_bf16", load().qdr_decode_step_bf16(
            self._h, _dptr(slots, torch.int32, "slots"), B,
            _dptr(q, bf, "q", B * H * DIM), _dptr(k, bf, "k", B * H * DIM),
            _dptr(v, bf, "v", B * H * DIM), _dptr(beta, f32, "beta", B * H),
            _dptr(gate, f32, "gate", gn), _dptr(o, bf, "o", B * H * DIM), _stream(stream)))

    def qdr_decode_step_split(self, slots, q, k, v, beta, gate, o, stream_readout=None, stream_writeback=None):
        import torch
        B, H = slots.numel(), self.num_heads
        f32 = torch.float32
        gn = B * H if self.gate == GATE_SCALAR else B * H * DIM
        _check("qdr_decode_step_split", load().qdr_decode_step_split(
            self._h, _dptr(slots, torch.int32, "slots"), B,
            _dptr(q, f32, "q", B * H * DIM), _dptr(k, f32, "k", B * H * DIM),
            _dptr(v, f32, "v", B * H * DIM), _dptr(beta, f32, "beta", B * H),
            _dptr(gate, f32, "gate", gn), _dptr(o, f32, "o", B * H * DIM),
            _stream(stream_readout), _stream(stream_writeback)))

    def qdr_read_raw(self, slot, stream=None) -> np.ndarray:
        out = np.empty(self.slot_stride, np.uint8)
        _check("qdr_read_raw", load().qdr_read_raw(
            self._h, int(slot), out.ctypes.data_as(ctypes.c_void_p), out.size, _stream(stream)))
        return out

    def qdr_write_raw(self, slot, data, stream=None):
        data = np.ascontiguousarray(data, np.uint8)
        _check("qdr_write_raw", load().qdr_write_raw(
            self._h, int(slot), data.ctypes.data_as(ctypes.c_void_p), data.size, _stream(stream)))

    def qdr_poll_device_error(self) -> int:
        f = ctypes.c_uint32(0)
        _check("qdr_poll_device_error", load().qdr_poll_device_error(self._h, ctypes.byref(f)))
        return int(f.value)

    # ---- helpers over the raw bytes of one block
    def block(self, raw_slot: np.ndarray, h: int) -> np.ndarray:
        off = int(self.head_off[h])
        return raw_slot[off: off + int(self.head_bytes[h])]


def qdr_last_error() -> str:
    return load().qdr_last_error().decode()
