"""PagedAttention decode for AMD Instinct MI355X (gfx950).

The decode itself runs in the HIP library ``libpadecode.so`` (C ABI declared
in ``include/pa_decode.h``); ``pa_decode`` below is its ctypes binding.
"""

from .binding import (PagedAttentionError, alloc_workspace, load_library, make_dims, pa_cache_append,  # noqa: F401
                      pa_cache_copy_blocks, pa_decode, plan, status_str, workspace_bytes)
