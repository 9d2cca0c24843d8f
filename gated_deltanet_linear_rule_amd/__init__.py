"""MI355X-native Gated DeltaNet (GDN) token mixer: C-ABI HIP library + thin binding.

The compute path is ``libgdn.so`` (hand-written HIP kernels for gfx950 behind
the C ABI declared in ``include/gdn.h``).  ``binding`` marshals torch tensors
into that ABI; there is no CPU fallback: calls fail loudly when the library is
missing.  ``inputs`` draws the seeded synthetic workloads.
"""
__all__ = ["gdn_prefill", "gdn_decode_step", "gdn_abi_version", "gdn_status_string"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
