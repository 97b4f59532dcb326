"""Shifted-chunk long-context attention for AMD MI355X (gfx950).

The compute lives in the HIP library ``libshattn.so`` (C-ABI, declared in
``include/shattn.h``); :mod:`.binding` marshals torch device tensors into it.
The library is loaded on first use, so the workload tables import without it.
"""

from .workloads import BY_NAME, WORKLOADS, Workload, gen_qkv, make_inputs  # noqa: F401


def __getattr__(name):
    if name in ("attn_chunk_fwd", "lse_merge", "attn_shifted_fwd", "attn_status_string",
                "ShattnError", "library_path", "load_library"):
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
