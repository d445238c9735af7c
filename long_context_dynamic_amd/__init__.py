"""MI355X (gfx950) Native Sparse Attention forward.

The work runs in libnsa.so (hand-written HIP, C ABI in include/nsa.h);
``long_context_dynamic_amd.nsa`` is its thin ctypes binding.
``workloads`` names the problem shapes and ``inputs`` makes seeded
synthetic inputs for them.
"""
__all__ = ["nsa", "workloads", "inputs"]
