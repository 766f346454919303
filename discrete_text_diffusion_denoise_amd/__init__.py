"""MI355X-native denoising step of a block text-diffusion MoE language model.

The compute path is the HIP library ``libdg.so`` (C ABI in include/dg.h);
``binding`` marshals torch tensors into it.  ``synthetic`` draws seeded inputs.
Importing this package loads nothing; ``binding.lib()`` loads the library and
raises if it has not been built.
"""
__all__ = ["binding", "synthetic"]
