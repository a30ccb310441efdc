"""MI355X-native frame-wise Gated DeltaNet forward (libsanawm_gdn + binding).

Importing the package loads nothing: the HIP library is opened on the first
call of ``gdn_fwd`` / ``gdn_chunk_step`` (see ``gdn.py``), and that call fails
loudly if the library is missing.
"""
__all__ = ["gdn_fwd", "gdn_chunk_step", "workspace_bytes", "GdnError"]


def __getattr__(name):
    if name in __all__:
        from . import gdn
        return getattr(gdn, name)
    raise AttributeError(name)
