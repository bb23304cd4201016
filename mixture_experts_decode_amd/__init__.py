"""MI355X-native small-batch decode MoE layer.

The hot path lives in ``libmoe_decode.so`` (hand-written HIP for gfx950 behind
a C ABI, declared in ``include/moe_decode.h``); ``moe_decode`` is its thin
ctypes binding and ``synth`` the seeded synthetic-layer generator.
"""
