"""zg_attn for MI355X: gated sliding-window + global causal attention (ZGCM-1).

The compute runs in the HIP library ``libzgattn.so`` built next to this file;
``global_attention_zg_amd.binding`` is the thin ctypes layer over its C ABI.
Importing this package loads nothing; the binding loads the library on first
use and raises if it is missing.
"""

__all__ = ["binding", "inputs"]


def __getattr__(name):
    if name in ("zg_attn_fwd", "zg_attn_decode", "zg_attn_fwd_workspace_size",
                "zg_attn_decode_workspace_size", "zg_attn_strerror", "ZgAttnError"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
