"""Fused tiled attention for AMD Instinct MI355X (gfx950).

Python face of the C-ABI library ``libattn.so`` (declared in
``include/attn.h``): argument marshalling only, every step of the
computation runs in the library's HIP kernels. The library is loaded on
first use; if it is missing or fails to load, every entry point raises.
"""

from ._binding import (  # noqa: F401
    AttnError,
    prefill,
    decode_paged,
    decode_paged_noalloc,
    DECODE_NOALLOC_SCRATCH_BYTES,
    decode_paged_workspace_size,
    paged_workspace_size,
    decode_paged_partition_size,
    kv_append,
    add_rmsnorm,
    status_string,
    library_path,
    load_library,
)
