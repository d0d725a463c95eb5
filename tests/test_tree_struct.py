"""Linked token trees <-> the flat arrays the C ABI takes."""
import numpy as np

import oracle
from token_tree_verification_02_amd import tree as T
from token_tree_verification_02_amd import workloads as W
from tests.test_oracle_pins import read_fig_tree


def test_fig_tree_flattens_to_bfs_labels():
    # the explainer's merged tree: Root -> A, B; A -> C, D; B -> E; C -> F; D -> G; E -> H
    n = {k: T.TreeNode(i) for i, k in enumerate("RABCDEFGH")}
    for p, c in ["RA", "RB", "AC", "AD", "BE", "CF", "DG", "EH"]:
        n[p].children.append(n[c])
    parent, depth, tokens, _ = T.flatten(n["R"])
    gp, gd, _ = read_fig_tree()
    assert list(parent) == list(gp) and list(depth) == list(gd)
    assert list(tokens) == list(range(9))
    assert oracle.validate_tree(parent, depth)


def test_roundtrip_random_trees():
    rng = np.random.default_rng(0)
    for _ in range(50):
        parent = W.random_tree(rng, int(rng.integers(1, 40)), 6)
        tokens = rng.integers(0, 1000, size=len(parent)).astype(np.int32)
        root = T.unflatten(parent, tokens)
        p2, d2, t2, _ = T.flatten(root)
        # flatten renumbers in BFS order; the multiset of root paths (as token strings) is preserved
        def paths(par, tok):
            out = set()
            for u in range(len(par)):
                out.add(tuple(int(tok[v]) for v in oracle.ancestors(par, u)[::-1]))
            return out
        assert paths(parent, tokens) == paths(p2, t2)
        assert oracle.validate_tree(p2, d2)
