"""MI355X-native paged KV-cache decode path (PagedAttention hot path).

The product is ``libpa.so`` (HIP kernels for gfx950 behind the C ABI of
``include/pa.h``); this package is its thin Python binding plus the build
script.  PyTorch provides device memory and streams only.
"""

from .binding import (  # noqa: F401
    EXPORTED,
    PA_DTYPE_BF16,
    PA_DTYPE_F32,
    PagedAttentionError,
    alloc_workspace,
    append_decode,
    append_decode_partials,
    copy_blocks,
    decode,
    decode_merge,
    decode_partials,
    decode_scratch,
    decode_shared_prefix,
    decode_shared_prefix_merge,
    decode_shared_prefix_workspace_bytes,
    alloc_shared_prefix_workspace,
    decode_workspace_bytes,
    empty_kv_cache,
    kv_cache_shapes,
    library_path,
    load_library,
    prefill,
    cp_slot_mapping,
    cp_context_lens,
    merge_states,
    map_to_kernel_blocks,
    slot_mapping,
    status_string,
    write_kv,
)
from .block_manager import (  # noqa: F401
    EXPORTED_BM,
    PA_ERR_NO_BLOCKS,
    PA_ERR_STATE,
    BlockManager,
)
