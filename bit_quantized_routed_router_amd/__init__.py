"""ds4moe: the routed mixture-of-experts layer of DeepSeek V4 Flash with 2-bit
quantized experts (CB2 gate/up, Q2K down), as hand-written HIP kernels for
AMD Instinct MI355X (gfx950) behind a C ABI.

    from bit_quantized_routed_router_amd import ds4moe     # ctypes binding
    from bit_quantized_routed_router_amd import synthetic  # seeded workloads

Importing the package loads nothing; ds4moe.lib() loads libds4moe.so and
raises if it has not been built.
"""
