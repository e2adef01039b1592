"""MI355X-native multi-LoRA SGMV delta path (segment build, plan, shrink, expand).

The compute lives in a HIP/C++ shared library (``csrc/``, C ABI declared in
``include/lora_sgmv.h``); ``binding`` is a thin ctypes layer over it with the
same function names.  Importing this package loads nothing: the library is
opened on first use by ``binding.lib()``, which raises if it has not been built.
"""
__all__ = ["binding", "workloads", "accounting"]
