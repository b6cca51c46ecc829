"""Paged grouped-query decode attention for MI355X (gfx950).

The work runs in a HIP C-ABI library (``libpa_decode.so``, declared in
``include/pa_decode.h``); this package only marshals torch tensors into it.
Importing the package loads nothing; the library is opened on first use and a
missing library raises instead of falling back to anything else.
"""

__all__ = ["append_kv", "decode_attention", "append_decode_attention", "decode_workspace_bytes",
           "validate_metadata", "status_string", "load_library"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
