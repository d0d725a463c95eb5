"""Token-tree verification hot path for MI355X (gfx950).

SpecInfer's tree attention (each tree node attends to the cached prefix plus its
own root path, in one pass), greedy tree verification and the commit of the
accepted path's keys and values to the cache, as hand-written HIP kernels behind
the C ABI in include/tree_verify.h, with the construction of the tree (top-k
expansion and merge of drafts) before it.  The functions here are the
ctypes binding of that library; torch provides device memory and streams.
"""
from ._lib import (TV_BF16, TV_EHIP, TV_EINVAL, TV_ETOPOLOGY, TV_EUNSUPPORTED, TV_EWORKSPACE,  # noqa: F401
                   TV_F16, TV_F32, TV_FP8_E4M3, TV_MERGE_MMAX, TV_MSS_VMAX, TV_NMAX, TV_NOALLOC_SCRATCH_BYTES, TV_OK,
                   TV_PAGE, TV_TOPK_MAX, TreeVerifyError, attn_desc, last_error, load,
                   tree_attention, tree_attention_noalloc, tree_build, tree_commit_kv, tree_expand_topk,
                   tree_merge_drafts,
                   tree_verify_greedy,
                   tree_verify_stochastic, stochastic_workspace_size, stochastic_set_poll_limit, validate_host,
                   workspace_size)
