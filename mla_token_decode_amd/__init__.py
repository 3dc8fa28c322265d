"""MLA speculative-verify decode for MI355X (gfx950).

The compute path is the C-ABI library ``libmla_decode.so`` (hand-written HIP
kernels, see ``include/mla_decode.h``); ``mla_token_decode_amd.binding`` is
its thin ctypes binding.  Importing this package loads nothing: the library
is opened on first use and a missing library is an error, never a fallback.
"""
__all__ = ["binding", "inputs"]
