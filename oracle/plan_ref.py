"""Candidate-tree plans (oracle side).

The glossary page "Medusa Heads", section "Attention arborescente et
acceptation": the best hypotheses of each head are combined as a Cartesian
product into candidate continuations that share prefixes and form a tree (its
example: top-2 of head 1 times top-3 of head 2 gives six candidates); the
authors found that a sparse 64-node tree built from the most accurate
combinations beats a dense 256-node tree.

A node is identified by its rank tuple (i_1, ..., i_d): the candidate at depth
d takes head d's rank-i_d token, under the parent (i_1, ..., i_{d-1}).  Node 0
is the root, the empty tuple, which carries the base model's own next token.
Readings where the page is silent (stated once, used everywhere):

* "most accurate combinations": a tuple's score is the product over its
  depths of the per-head rank accuracy acc[d-1][i_d]; the sparse tree keeps the
  N-1 best tuples ordered by (score descending, depth ascending, tuple
  lexicographically ascending), plus the root.
* nodes are stored in breadth-first order: depth ascending, then tuple
  lexicographically ascending.
* "sees only its ancestors": a node attends to its ancestors and to itself.

Pins (CPU tests): the closed-form node count 1 + sum_d prod_{k<=d} s_k of full
trees (9 nodes / 6 leaves for the page's 2x3 example, 256 for 3x4x4x4); mask
popcount = depth + 1; prefix closure of sparse plans; brute force over all
prefix-closed subsets of tiny Cartesian trees showing the greedy selection has
the largest total score.
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

__all__ = ["TreePlan", "plan_from_paths", "plan_full", "plan_from_accuracy", "candidate_tuples"]


@dataclass
class TreePlan:
    paths: List[Tuple[int, ...]]   # breadth-first; paths[0] == ()
    parent: np.ndarray             # [N] int32, -1 for the root
    depth: np.ndarray              # [N] int32
    rank: np.ndarray               # [N] int32, rank within its head's top-k; -1 for the root
    anc: np.ndarray                # [N, N] bool: anc[i, j] <=> j is an ancestor of i or j == i

    @property
    def n_nodes(self) -> int:
        return len(self.paths)

    @property
    def max_depth(self) -> int:
        return int(self.depth.max()) if len(self.paths) else 0

    @property
    def mask_words(self) -> int:
        return (self.n_nodes + 63) // 64

    def mask_bits(self) -> np.ndarray:
        """[N, mask_words] uint64; bit j of row i set <=> anc[i, j]."""
        W = self.mask_words
        out = np.zeros((self.n_nodes, W), dtype=np.uint64)
        for i in range(self.n_nodes):
            for j in np.nonzero(self.anc[i])[0]:
                out[i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
        return out

    def leaves(self) -> List[int]:
        has_child = np.zeros(self.n_nodes, dtype=bool)
        has_child[self.parent[self.parent >= 0]] = True
        return [i for i in range(self.n_nodes) if not has_child[i]]

    def path_nodes(self, i: int) -> List[int]:
        """Node indices from the root down to node i."""
        out = []
        while i >= 0:
            out.append(i)
            i = int(self.parent[i])
        return out[::-1]


def plan_from_paths(paths: Sequence[Sequence[int]]) -> TreePlan:
    """Build a plan from candidate rank tuples (the root is added).

    Rejects duplicate tuples, negative ranks and sets that are not closed under
    taking prefixes (every candidate's parent must itself be a candidate)."""
    tups = [tuple(int(x) for x in p) for p in paths]
    if any(len(t) == 0 for t in tups):
        raise ValueError("the root is implicit; do not list the empty tuple")
    if len(set(tups)) != len(tups):
        raise ValueError("duplicate candidate tuple")
    if any(x < 0 for t in tups for x in t):
        raise ValueError("negative rank")
    present = set(tups)
    for t in tups:
        if len(t) > 1 and t[:-1] not in present:
            raise ValueError(f"tuple {t} has no parent {t[:-1]}")
    order = [()] + sorted(tups, key=lambda t: (len(t), t))
    index = {t: i for i, t in enumerate(order)}
    N = len(order)
    parent = np.full(N, -1, dtype=np.int32)
    depth = np.zeros(N, dtype=np.int32)
    rank = np.full(N, -1, dtype=np.int32)
    anc = np.zeros((N, N), dtype=bool)
    for i, t in enumerate(order):
        depth[i] = len(t)
        if t:
            parent[i] = index[t[:-1]]
            rank[i] = t[-1]
        for d in range(len(t) + 1):
            anc[i, index[t[:d]]] = True
    return TreePlan(paths=order, parent=parent, depth=depth, rank=rank, anc=anc)


def candidate_tuples(tree_s: Sequence[int]) -> List[Tuple[int, ...]]:
    """Every rank tuple of the Cartesian product of the per-depth top-k sizes,
    for depths 1..len(tree_s)."""
    out: List[Tuple[int, ...]] = []
    for d in range(1, len(tree_s) + 1):
        out.extend(itertools.product(*[range(int(s)) for s in tree_s[:d]]))
    return out


def plan_full(tree_s: Sequence[int]) -> TreePlan:
    """The dense tree: the full Cartesian product at every depth."""
    return plan_from_paths(candidate_tuples(tree_s))


def plan_from_accuracy(acc: np.ndarray, tree_s: Sequence[int], n_nodes: int) -> TreePlan:
    """Sparse tree of ``n_nodes`` nodes (root included) from the most accurate
    combinations: score(t) = prod_d acc[d-1][t_d]; keep the best n_nodes-1."""
    cands = candidate_tuples(tree_s)
    if n_nodes - 1 > len(cands):
        raise ValueError("more nodes requested than candidate tuples exist")

    def score(t):
        p = 1.0
        for d, r in enumerate(t):
            p *= float(acc[d][r])
        return p

    ranked = sorted(cands, key=lambda t: (-score(t), len(t), t))
    return plan_from_paths(ranked[: n_nodes - 1])
