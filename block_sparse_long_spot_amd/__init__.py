"""SpotAttention decode hot path on MI355X (gfx950): HIP kernels behind a C ABI.

The functions below are thin bindings to libspot.so with the C entry points' names;
see include/spot.h for the contract of each.
"""
from ._lib import (  # noqa: F401
    SPOT_BF16,
    SPOT_F32,
    SPOT_FP4_E2M1_G32,
    SPOT_FP8_E4M3,
    SPOT_INT4_G32,
    SPOT_INT8,
    Prepared,
    SpotError,
    load,
    selector_format,
    spot_abi_version,
    spot_prefill_attn,
    spot_prefill_select_score,
    spot_prefill_select_topp,
    spot_quantize_selector,
    spot_select_score,
    spot_select_topp,
    spot_sparse_attn,
    spot_sparse_attn_noalloc,
    spot_sparse_attn_workspace_bytes,
    status_string,
)
from .decode import DecodeStep, decode_step  # noqa: F401
