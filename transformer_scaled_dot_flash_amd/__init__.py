"""Scaled dot-product attention forward for AMD MI355X (gfx950).

* ``attn``       ctypes binding of the C ABI (include/attn.h), same names.
* ``ops_torch``  torch front end (allocation and streams only).
* ``inputs``     seeded synthetic N(0,1) inputs.
* ``workloads``  the benchmark/parity workloads and their work counts.
"""
from .attn import (ATTN_BF16, ATTN_F32, AttnError, attn_abi_version, attn_fwd_decode,
                   attn_fwd_decode_default_splits, attn_fwd_decode_workspace_bytes,
                   attn_fwd_prefill, attn_last_hip_error, attn_status_string, load_library)

__all__ = [
    "ATTN_BF16", "ATTN_F32", "AttnError", "attn_abi_version", "attn_fwd_decode",
    "attn_fwd_decode_default_splits", "attn_fwd_decode_workspace_bytes", "attn_fwd_prefill",
    "attn_last_hip_error", "attn_status_string", "load_library",
]
