"""MI355X-native fused packed low-bit BitLinear product (i2_s, TQ2_0, W1A8).

The compute path is the C-ABI library ``liblowbit.so`` (hand-written HIP for
gfx950, declared in ``include/lowbit.h``); :mod:`binary_bit_weight_amd.lowbit`
is its ctypes binding.  Importing this package loads nothing; the library is
loaded on first use and a missing build raises instead of falling back.
"""
__all__ = ["lowbit", "synth", "build"]
