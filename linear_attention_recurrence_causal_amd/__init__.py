"""MI355X-native Gated DeltaNet core: C-ABI library of HIP kernels + thin binding.

``gdn`` (the binding) is imported lazily so that the input generators can be
used on machines without the built library.
"""
__all__ = ["gdn", "inputs"]
