"""Token trees as linked nodes, and their flat form for the C ABI.

The SpecInfer explainer (tree-verification section) represents a speculated
token tree as nodes that carry a draft token id, the small model's probability
of it, and a list of children.  The library takes the same tree as flat arrays
in a topological order: node 0 is the root, parent[u] < u.  `flatten` produces
them in breadth-first order; `unflatten` rebuilds the linked form.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class TreeNode:
    token_id: int
    ssm_prob: float = 1.0
    children: list["TreeNode"] = field(default_factory=list)


def flatten(root: TreeNode):
    """(parent, depth, tokens, ssm_prob) arrays of the tree in BFS order (root = node 0)."""
    parent, depth, tokens, probs = [-1], [0], [root.token_id], [root.ssm_prob]
    queue = [(root, 0)]
    head = 0
    while head < len(queue):
        node, idx = queue[head]
        head += 1
        for ch in node.children:
            parent.append(idx)
            depth.append(depth[idx] + 1)
            tokens.append(ch.token_id)
            probs.append(ch.ssm_prob)
            queue.append((ch, len(parent) - 1))
    return (np.array(parent, np.int32), np.array(depth, np.int32), np.array(tokens, np.int32),
            np.array(probs, np.float32))


def unflatten(parent, tokens, probs=None) -> TreeNode:
    """Linked nodes from flat arrays in a topological order."""
    n = len(parent)
    nodes = [TreeNode(int(tokens[u]), 1.0 if probs is None else float(probs[u])) for u in range(n)]
    for u in range(1, n):
        nodes[int(parent[u])].children.append(nodes[u])
    return nodes[0]
