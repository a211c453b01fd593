"""MI355X-native NF4 QLoRA linear layer.

The compute lives in ``libnf4qlora.so`` (hand-written HIP kernels for gfx950
behind a C ABI declared in ``include/nf4qlora.h``).  ``nf4qlora`` is the thin
ctypes binding; importing it loads the library and fails loudly when it has
not been built.  ``workloads`` draws the seeded synthetic inputs.
"""
__all__ = ["nf4qlora", "workloads"]
