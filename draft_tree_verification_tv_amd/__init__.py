"""Tree verification for speculative decoding on AMD Instinct MI355X (gfx950).

The compute lives in ``libtv.so`` (hand-written HIP, C ABI in ``include/tv.h``); this
package is its thin Python binding.
"""

from .tv import (  # noqa: F401
    EXPORTS,
    HEAD_DIM,
    MAX_NODES,
    NOALLOC_SCRATCH_BYTES,
    TV_ERR_WORKSPACE,
    TVError,
    abi_version,
    accept,
    argmax,
    argmax_accept,
    argmax_workspace,
    argmax_workspace_size,
    kv_commit,
    kv_quantize_fp8,
    kv_quantize_mx4,
    tree_attn_mx4,
    lib,
    sample_accept,
    status_string,
    tree_attn,
    tree_attn_fp8,
    tree_attn_noalloc,
    tree_attn_workspace_size,
    tree_prep,
    validate_tree_host,
    verify,
)
