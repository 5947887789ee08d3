"""The node budget (glossary "Medusa Heads", section "Attention arborescente et acceptation":
a sparse tree of the most accurate combinations; 64 such nodes beat a 256-node dense tree).

The library's expected accepted length is pinned by exact enumeration of every outcome of
the heads (each head independently right at one rank, or at none), the sparse choice by
brute force over every prefix-closed node set of small Cartesian trees.  Host only."""
import itertools
import os
import re

import numpy as np
import pytest

from speculative_decoding_amd import budget
from speculative_decoding_amd import medusa as M

HERE = os.path.dirname(os.path.abspath(__file__))


def _acc(seed, widths, cols=None):
    """Random descending per-head rank accuracies whose rows sum below 1."""
    g = np.random.default_rng(seed)
    cols = cols or max(widths)
    acc = np.zeros((len(widths), cols))
    for d, w in enumerate(widths):
        p = np.sort(g.dirichlet(np.ones(w + 1))[:w])[::-1]
        acc[d, :w] = p * g.uniform(0.5, 1.0)
    return acc


def _enumerated_accept(plan, acc, widths):
    """E[accepted length] by summing over every joint outcome of the heads: head d's right
    token sits at rank r (probability acc[d][r]) or outside its list (the rest).  The
    accepted length of an outcome is the deepest prefix of its ranks that is a tree node."""
    parent, depth, rank, _ = plan.arrays()
    nodes = set()
    for i in range(1, len(parent)):
        t, j = [], i
        while j > 0:
            t.append(int(rank[j]))
            j = int(parent[j])
        nodes.add(tuple(reversed(t)))
    D = len(widths)
    total = 0.0
    for outcome in itertools.product(*[list(range(w)) + [None] for w in widths]):
        p = 1.0
        for d, r in enumerate(outcome):
            p *= acc[d, r] if r is not None else 1.0 - acc[d, : widths[d]].sum()
        a = 0
        for d in range(1, D + 1):
            t = outcome[:d]
            if None in t or t not in nodes:
                break
            a = d
        total += p * a
    return total


@pytest.mark.parametrize("widths,seed", [((3, 2, 2), 0), ((4, 3), 1), ((2, 2, 2, 2), 2),
                                         ((5,), 3)])
def test_expected_accept_equals_enumeration(widths, seed):
    acc = _acc(seed, widths, cols=6)
    n_cands = sum(int(np.prod(widths[:d])) for d in range(1, len(widths) + 1))
    plans = [M.medusa_tree_plan_full(widths)]
    plans += [M.medusa_tree_plan_from_accuracy(acc, widths, n) for n in (1, 2, 3, n_cands // 2 + 1,
                                                                         n_cands + 1)]
    # a hand-picked tree that is neither full nor the most accurate choice
    plans.append(M.medusa_tree_plan_create([(widths[0] - 1,)] + ([(widths[0] - 1, 0)]
                                           if len(widths) > 1 else [])))
    for plan in plans:
        want = _enumerated_accept(plan, acc, widths)
        got = plan.expected_accept(acc)
        assert abs(got - want) < 1e-12, (plan.info(), got, want)


def _downsets(widths):
    """Every prefix-closed set of rank tuples of the Cartesian tree of ``widths``."""
    def sub(prefix):
        d = len(prefix)
        if d == len(widths):
            return [[]]
        per_child = []
        for r in range(widths[d]):
            t = prefix + (r,)
            per_child.append([[]] + [[t] + rest for rest in sub(t)])
        out = []
        for combo in itertools.product(*per_child):
            out.append([x for part in combo for x in part])
        return out
    return sub(())


@pytest.mark.parametrize("widths,seed", [((3, 2, 2), 4), ((2, 3, 2), 5)])
def test_sparse_choice_maximises_expected_accept(widths, seed):
    acc = _acc(seed, widths)
    best = {}
    for ds in _downsets(widths):
        e = sum(np.prod([acc[d, r] for d, r in enumerate(t)]) for t in ds)
        best[len(ds)] = max(best.get(len(ds), -1.0), e)
    assert len(best) == max(best) + 1
    for n_paths, e in best.items():
        got = M.medusa_tree_plan_from_accuracy(acc, widths, n_paths + 1).expected_accept(acc)
        assert abs(got - e) < 1e-12, (n_paths, got, e)


def test_root_only_and_monotone():
    acc = _acc(6, (10, 5, 4, 4))
    pts = budget.curve(acc, (10, 5, 4, 4), [1, 2, 16, 64, 256, 341, 1024], dense=[(3, 4, 4, 4)])
    sparse = [p for p in pts if p.kind == "sparse"]
    assert sparse[0].nodes == 1 and sparse[0].expected_accept == 0.0 and sparse[0].max_depth == 0
    e = [p.expected_accept for p in sparse]
    assert all(b >= a for a, b in zip(e, e[1:]))
    assert pts[-1].kind == "dense" and pts[-1].nodes == 256
    # the sparse choice is the best tree of its size, so 256 sparse nodes beat the dense 256
    assert sparse[4].nodes == 256 and sparse[4].expected_accept >= pts[-1].expected_accept


def test_sparse64_beats_dense256_on_the_synthetic_table():
    """The page's ordering reproduced on the sweep's synthetic accuracy table (the 8B
    shape's heads with the last head widened to four ranks so the dense tree exists)."""
    import dataclasses
    from synth import get_config
    from synth.gen import accuracy_table
    s = (10, 5, 4, 4)
    acc = accuracy_table(dataclasses.replace(get_config("8b"), s=s, tree_s=s), 0)
    e64 = M.medusa_tree_plan_from_accuracy(acc, s, 64).expected_accept(acc)
    e256 = M.medusa_tree_plan_full((3, 4, 4, 4)).expected_accept(acc)
    assert e64 > e256


def test_best_budget():
    pts = [budget.BudgetPoint("sparse", 1, 0, 0.0, 1e-3),
           budget.BudgetPoint("sparse", 64, 4, 1.6, 1.0e-3),
           budget.BudgetPoint("sparse", 128, 4, 1.6, 1.0e-3),
           budget.BudgetPoint("dense", 256, 4, 1.59, 2e-3)]
    b = budget.best(pts)
    assert b.nodes == 64 and abs(b.tokens_per_s - 2600.0) < 1e-6
    with pytest.raises(ValueError):
        budget.best([budget.BudgetPoint("sparse", 1, 0, 0.0)])


def test_expected_accept_rejects_short_table():
    plan = M.medusa_tree_plan_full((2, 2, 2))
    with pytest.raises(M.MedusaError):
        plan.expected_accept(np.full((2, 2), 0.3))      # three levels, two rows
    with pytest.raises(M.MedusaError):
        plan.expected_accept(np.full((3, 1), 0.3))      # rank 1 used, one column


def test_limit_constants_match_header():
    text = open(os.path.join(HERE, "..", "include", "medusa.h")).read()
    for name in ("MEDUSA_MAX_TOPK", "MEDUSA_MAX_HEADS", "MEDUSA_MAX_NODES",
                 "MEDUSA_NOALLOC_SCRATCH_BYTES"):
        v = int(re.search(rf"#define {name} (\d+)", text).group(1))
        assert getattr(M, name) == v, name
