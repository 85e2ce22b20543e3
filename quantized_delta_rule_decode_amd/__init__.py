"""MI355X-native quantized gated delta-rule decode step.

The compute path lives in ``libqdr.so`` (HIP kernels for gfx950 behind a
C ABI declared in ``include/qdr.h``); ``qdr`` is its thin Python binding.
"""
from . import synth  # noqa: F401

__all__ = ["synth", "qdr"]


def __getattr__(name):
    if name == "qdr":
        from . import qdr as _qdr
        return _qdr
    raise AttributeError(name)
