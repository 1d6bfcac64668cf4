"""MI355X-native GPT-2 pre-training step: HIP kernels for gfx950 behind a C ABI.

``lib.GPT2Step`` binds one context of libgpt2.so with PyTorch-owned device
buffers; ``build.build()`` compiles the library in-tree.
"""

__all__ = ["lib", "build"]
