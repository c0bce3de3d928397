"""Exact tiled attention over a paged KV cache for AMD MI355X (gfx950).

The compute path is the HIP library libpagedattn.so (C ABI in include/pagedattn.h);
`binding` wraps it with ctypes.  `workloads` draws seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    EXPORTED, ContractError, KVLayout, PagedAttnError, PreparedDecode, PreparedPrefill,
    contract_violations,
    decode_workspace,
    last_error, layout_of, set_contract_check,
    load_library, make_layout, pa_decode, pa_decode_combine, pa_decode_partial,
    pa_decode_split_tokens, pa_decode_workspace_bytes, pa_prefill, status_string,
)

__version__ = "0.1.0"
