"""libmoe: fused Mixture-of-Experts layer forward for MI355X (gfx950).

The compute lives in the HIP library ``libmoe.so`` built from ``csrc/``; this
package only marshals arguments to its C ABI (see ``_binding``).  Importing the
package does not load the library; the first call through ``lib()`` does, and
fails loudly if it is missing.
"""
__all__ = ["lib", "roofline"]


def lib():
    from . import _binding
    return _binding.load()
