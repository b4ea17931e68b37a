"""MI355X (gfx950) paged MLA cache write and split-KV MLA decode.

The compute runs in the HIP library ``libmla_amd.so`` built from ``csrc/``;
the functions here only marshal torch tensors into its C ABI.  The library is
loaded on first use; there is no CPU fallback.
"""

from .binding import (  # noqa: F401
    MLAError,
    cache_write,
    decode,
    decode_noalloc,
    decode_workspace_bytes,
    library_path,
    linear,
    linear_workspace_bytes,
    load_library,
    merge_partials,
    num_kv_splits,
    rope_q,
)
