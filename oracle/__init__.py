"""CPU oracle (test infrastructure only; see tree_oracle)."""
from .tree_oracle import (TV_EINVAL, TV_ETOPOLOGY, TV_OK, accept_walk, ancestors, argmax_lowest,  # noqa: F401
                          cache_values, commit_kv, expand_topk, fp8_e4m3_value, gather_prefix, merge_drafts, mss_walk, softmax64, to_f64, tree_attention, tree_build,
                          topk_lowest, validate_tree, verify_greedy, verify_stochastic)
