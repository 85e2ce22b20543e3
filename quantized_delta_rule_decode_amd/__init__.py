"""MI355X-native quantized gated delta-rule decode step.

The compute path lives in ``libqdr.so`` (HIP kernels for gfx950 behind the C
ABI declared in ``include/qdr.h``); ``quantized_delta_rule_decode_amd.qdr``
is its thin Python binding, ``synth`` the seeded synthetic workloads and
``workload`` the device-side pool set-up used by the benchmark.
"""
