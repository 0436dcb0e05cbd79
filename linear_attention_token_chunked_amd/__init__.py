"""MI355X-native Gated DeltaNet (GDN) token mixer.

The compute path is the HIP library ``libgdn.so`` (gfx950 kernels behind a C
ABI declared in ``include/gdn.h``); ``linear_attention_token_chunked_amd.gdn``
is its thin ctypes binding.  ``inputs`` draws seeded synthetic workloads.
The binding is imported lazily so that ``inputs`` can be used without the
built library.
"""

__all__ = ["fwd_chunked", "decode_step", "inputs"]


def __getattr__(name):
    if name in ("fwd_chunked", "decode_step", "fwd_chunked_workspace_size", "lib"):
        from . import gdn

        return getattr(gdn, name)
    raise AttributeError(name)
