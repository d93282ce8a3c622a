"""MI355X-native block-sparse causal attention with learned block selection.

The compute path is the HIP library ``libsparse_attn.so`` (built from
``csrc/`` for gfx950) behind a C ABI declared in ``include/sparse_attn.h``;
``ops`` is a thin ctypes binding with the same entry-point names.  Importing
this package loads nothing: ``ops`` loads the library on first use and raises
if it is missing.
"""

__all__ = ["ops", "inputs"]
