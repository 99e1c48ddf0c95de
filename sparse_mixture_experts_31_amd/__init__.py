"""Mixtral sparse-MoE feed-forward layer for one AMD MI355X (gfx950).

The layer runs in hand-written HIP kernels behind the C ABI of
``libmoe.so`` (declared in ``include/moe.h``); ``moe`` is the thin Python
binding over it and ``inputs`` draws the seeded synthetic workloads.
"""
