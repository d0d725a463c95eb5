"""CPU oracle (test infrastructure only; see tree_oracle)."""
from .tree_oracle import (TV_EINVAL, TV_ETOPOLOGY, TV_OK, accept_walk, ancestors, argmax_lowest,  # noqa: F401
                          commit_kv, gather_prefix, mss_walk, softmax64, to_f64, tree_attention, tree_build,
                          validate_tree, verify_greedy, verify_stochastic)
