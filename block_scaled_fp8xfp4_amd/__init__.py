"""Block-scaled routed-expert MoE layer and dense block-32 FP8 projection for
AMD Instinct MI355X (gfx950).

The computation lives in libmxmoe.so (HIP kernels behind the C-ABI declared in
include/mxmoe.h).  ``mxmoe`` is its ctypes binding, ``layer`` a convenience
wrapper that owns workspaces, ``synth`` the seeded workload generator.
Nothing here falls back to a CPU or PyTorch implementation.
"""
