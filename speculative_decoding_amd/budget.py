"""Node budget of the candidate tree: how many nodes a step should verify.

The glossary page "Medusa Heads" (section "Attention arborescente et acceptation") builds
the sparse tree from the most accurate combinations of the heads' candidates and reports
that 64 such nodes beat a 256-node dense tree.  With per-head rank accuracies
acc[d-1][r] (the probability that head d's rank-r candidate is the base model's next
token) and independent heads, a node is accepted with the product of acc along its path,
and siblings exclude one another, so the expected accepted length E[a](N) of an N-node
tree is the sum of those products (``TreePlan.expected_accept``, computed by the library).
A step that takes t(N) seconds then emits (1 + E[a](N)) / t(N) tokens per second per
sequence: the accepted candidates plus the bonus token.  E[a] grows ever more slowly with
N while t(N) grows with the verified rows, so the best budget is where the ratio peaks.

Host logic only: the timing function is supplied by the caller (a function of a plan
that returns seconds per step), so this module launches nothing itself.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Iterable, List, Optional, Sequence

import numpy as np

from . import medusa as M


@dataclass
class BudgetPoint:
    kind: str                   # "sparse" (most accurate combinations) or "dense" (Cartesian)
    nodes: int                  # tree nodes including the root
    max_depth: int
    expected_accept: float      # E[a] under the accuracy table
    step_s: Optional[float] = None

    @property
    def tokens_per_step(self) -> float:
        return 1.0 + self.expected_accept

    @property
    def tokens_per_s(self) -> Optional[float]:
        """Predicted tokens/s per sequence: (1 + E[a]) / t(N)."""
        return None if not self.step_s else self.tokens_per_step / self.step_s

    def as_dict(self) -> dict:
        return {"kind": self.kind, "nodes": self.nodes, "max_depth": self.max_depth,
                "expected_accept_len": self.expected_accept,
                "ms_per_step": None if self.step_s is None else 1e3 * self.step_s,
                "tokens_per_step": self.tokens_per_step,
                "tokens_per_s_per_seq": self.tokens_per_s}


def plans(acc: np.ndarray, tree_s: Sequence[int], node_counts: Iterable[int],
          dense: Sequence[Sequence[int]] = ()):
    """(kind, plan) for every sparse budget in node_counts, then the full Cartesian tree of
    each per-depth branching in `dense`."""
    out = [("sparse", M.medusa_tree_plan_from_accuracy(acc, tree_s, int(n))) for n in node_counts]
    out += [("dense", M.medusa_tree_plan_full(ds)) for ds in dense]
    return out


def curve(acc: np.ndarray, tree_s: Sequence[int], node_counts: Iterable[int],
          step_seconds: Optional[Callable[[M.TreePlan], float]] = None,
          dense: Sequence[Sequence[int]] = ()) -> List[BudgetPoint]:
    """E[a] for each budget (and each dense tree), with t(N) from ``step_seconds`` when given."""
    pts = []
    for kind, plan in plans(acc, tree_s, node_counts, dense):
        n, depth, _ = plan.info()
        p = BudgetPoint(kind=kind, nodes=n, max_depth=depth,
                        expected_accept=plan.expected_accept(acc))
        if step_seconds is not None:
            p.step_s = float(step_seconds(plan))
        pts.append(p)
    return pts


def best(points: Sequence[BudgetPoint]) -> BudgetPoint:
    """The budget with the highest predicted tokens/s (fewest nodes on a tie)."""
    timed = [p for p in points if p.tokens_per_s is not None]
    if not timed:
        raise ValueError("no timed budget")
    return max(timed, key=lambda p: (p.tokens_per_s, -p.nodes))
