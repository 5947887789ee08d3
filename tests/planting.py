"""Planting: turn a random draw into inputs with wide decision margins and a
chosen acceptance pattern.  Test infrastructure; it calls the oracle only.

Random heads would never predict the greedy continuation, so every step would
accept nothing.  Planting edits a few weight rows so that

* head k ranks the greedy token g_{k+1} at the rank drawn for it from the
  synthetic accuracy table (or outside its top-s_k, for a drawn miss), by
  swapping two rows of that head's vocabulary projection;
* every discrete decision of the step has a margin of at least ``thr`` in
  fp64 on the final bits: the root argmax, each greedy step's argmax, the gaps
  among each head's top-(s_k + 1) logits, and the argmax at every tree node.
  Margins are opened by moving single weights by whole bf16 ulps along the
  direction of the hidden vector that decision reads (fp32 rows are moved
  directly).

If a draw cannot be fixed (the root or greedy chain itself is too close) the
last hidden state is re-drawn (``h_attempt``).  The result is a patch
(``synth.gen.apply_patch`` format); the generator applies it as plain data.
"""
from __future__ import annotations

import json
from dataclasses import dataclass
from typing import Dict, List, Optional, Tuple

import numpy as np

import oracle
from synth import make_inputs, get_config
from synth.gen import apply_patch

THR = 0.02        # margin required by the planting itself (tests assert >= 1e-2)
SPACING = 0.03    # gap the fixes aim for


def plan_for(cfg, acc) -> oracle.TreePlan:
    if cfg.tree == "full":
        return oracle.plan_full(cfg.tree_s)
    return oracle.plan_from_accuracy(acc, cfg.tree_s, cfg.n_nodes)


def margin_top1(logits: np.ndarray) -> float:
    t = np.partition(logits, -2)[-2:]
    return float(t[1] - t[0])


def expected_accept_len(plan: oracle.TreePlan, ranks: np.ndarray) -> int:
    """Deepest d such that (ranks[0..d)) is a node of the plan and no rank is a miss."""
    present = set(plan.paths)
    a = 0
    for d in range(1, plan.max_depth + 1):
        t = tuple(int(r) for r in ranks[:d])
        if any(r < 0 for r in t) or t not in present:
            break
        a = d
    return a


# ------------------------------------------------------------------ row edits

class _Editor:
    """Records edits to the generator's tensors and applies them in place."""

    def __init__(self, inp):
        self.inp = inp
        self.ops: List[dict] = []
        self.bf16 = inp.dtype == "bf16"

    def _mat(self, tensor: str, head: int) -> np.ndarray:
        return self.inp.w2[head] if tensor == "w2" else getattr(self.inp, tensor)

    def row_f64(self, tensor: str, head: int, r: int) -> np.ndarray:
        return oracle.as_f64(self._mat(tensor, head)[r], self.inp.dtype)

    def swap(self, tensor: str, head: int, a: int, b: int) -> None:
        op = {"op": "swap_rows", "tensor": tensor, "head": int(head), "a": int(a), "b": int(b)}
        apply_patch(self.inp, {"ops": [op]})
        self.ops.append(op)

    def move(self, tensor: str, head: int, r: int, x: np.ndarray, target: float,
             tol: float = 2e-3) -> None:
        """Move row r's dot product with x to ``target`` (within ``tol``)."""
        m = self._mat(tensor, head)
        if not self.bf16:
            row = self.row_f64(tensor, head, r)
            cur = float(row @ x)
            new = (row + (target - cur) * x / float(x @ x)).astype(np.float32)
            op = {"op": "set_row", "tensor": tensor, "head": int(head), "row": int(r),
                  "values": [float(v) for v in new]}
            apply_patch(self.inp, {"ops": [op]})
            self.ops.append(op)
            return
        total = np.zeros(m.shape[1], dtype=np.int32)
        for _ in range(12):
            bits = m[r].astype(np.int32)
            w = oracle.as_f64(m[r], "bf16")
            cur = float(w @ x)
            need = target - cur
            if abs(need) <= tol:
                break
            up = np.sign(need) * np.sign(x) > 0          # raise w_i where that helps
            # one ulp in the wanted direction: for w > 0 raising is bits+1, for w < 0 bits-1
            step = np.where(up == (w > 0), 1, -1)
            ok = (np.abs(w) > 2.0 ** -100) & (x != 0)
            nb = bits + step
            nw = oracle.as_f64(np.clip(nb, 0, 0xFFFF).astype(np.uint16), "bf16")
            gain = (nw - w) * x * np.sign(need)
            gain = np.where(ok & (gain > 0), gain, 0.0)
            order = np.argsort(-gain, kind="stable")
            cum = np.cumsum(gain[order])
            n = int(np.searchsorted(cum, abs(need) - tol * 0.5)) + 1
            n = min(n, int((gain > 0).sum()))
            if n <= 0:
                break
            cols = order[:n]
            m[r, cols] = (bits[cols] + step[cols]).astype(np.uint16)
            total[cols] += step[cols]
        cols = np.nonzero(total)[0]
        if len(cols):
            self.ops.append({"op": "add_bits", "tensor": tensor, "head": int(head), "row": int(r),
                             "cols": [int(c) for c in cols], "delta": [int(total[c]) for c in cols]})


# ------------------------------------------------------------------ checks

@dataclass
class Decision:
    kind: str          # "root", "chain", "node", "head"
    where: tuple
    margin: float


def head_gaps(logits: np.ndarray, s: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-(s+1) ids and the s gaps between consecutive ones."""
    ids = oracle.topk(logits, s + 1)
    v = logits[ids]
    return ids, v[:-1] - v[1:]


def all_decisions(inp, plan, res: "oracle.StepResult", chain_logits) -> List[Decision]:
    cfg = inp.cfg
    out = []
    for b in range(cfg.B):
        out.append(Decision("root", (b,), margin_top1(res.root_logits[b])))
        for j, lg in enumerate(chain_logits[b]):
            out.append(Decision("chain", (b, j), margin_top1(lg)))
        for i in range(plan.n_nodes):
            out.append(Decision("node", (b, i), margin_top1(res.logits[b, i])))
        for k in range(cfg.K):
            _, gaps = head_gaps(res.head_logits[b, k], cfg.s[k])
            out.append(Decision("head", (b, k), float(gaps.min())))
    return out


# ------------------------------------------------------------------ planting

def _greedy_chain(inp, plan, root: np.ndarray):
    """Greedy tokens g_1..g_{D+1} after the root, with their logits."""
    D = plan.max_depth
    toks, lgs = [], []
    for b in range(inp.cfg.B):
        t, _, lg = oracle.greedy_decode(inp, b, int(root[b]), D + 1)
        toks.append(t)
        lgs.append(lg)
    return toks, lgs


def _fix_one_head(ed: _Editor, inp, k: int, b: int, lg: np.ndarray, u: np.ndarray,
                  g: int) -> bool:
    """One repair of head k for sequence b; True if something was edited."""
    cfg = inp.cfg
    sk = cfg.s[k]
    rho = int(inp.plant_rank[b, k]) if g >= 0 else None
    order = oracle.topk(lg, sk + 200)
    pos = np.nonzero(order == g)[0]
    cur_rank = int(pos[0]) if len(pos) else None
    if rho is not None and rho >= 0 and cur_rank != rho:
        ed.swap("w2", k, g, int(order[rho]))
        return True
    if rho is not None and rho < 0 and cur_rank is not None and cur_rank <= sk:
        ed.swap("w2", k, g, int(order[sk + 100 + cur_rank]))
        return True
    ids, gaps = head_gaps(lg, sk)
    if gaps.min() >= THR:
        return False
    vals = lg[ids]
    targets = [float(vals[0])]
    for i in range(1, sk):
        targets.append(min(float(vals[i]), targets[-1] - SPACING))
    for i in range(1, sk):
        if targets[i] < float(vals[i]) - 1e-12:
            ed.move("w2", k, int(ids[i]), u, targets[i])
    limit = targets[-1] - SPACING
    for r in oracle.topk(lg, sk + 64)[sk:]:
        if lg[r] > limit:
            ed.move("w2", k, int(r), u, limit - 0.01)
    return True


def _fix_heads(ed: _Editor, inp, plan, chain, max_passes: int = 40) -> bool:
    """Plant the greedy tokens and open the top-k gaps of every head.  Each pass
    repairs at most one sequence per head (edits to a shared row move the other
    sequences' logits too), then re-evaluates."""
    cfg = inp.cfg
    _, _, _, u = oracle.heads_forward(inp.h, inp.w1, inp.b1, inp.w2, cfg.s, inp.dtype)
    for _ in range(max_passes):
        changed = False
        for k in range(cfg.K):
            for b in range(cfg.B):
                lg = oracle.matvec_rows(inp.w2[k], u[b, k], inp.dtype)
                g = int(chain[b][k]) if k < len(chain[b]) else -1
                if _fix_one_head(ed, inp, k, b, lg, u[b, k], g):
                    changed = True
                    break
        if not changed:
            return True
    return False


def plant(cfg, seed: int, max_attempts: int = 12, verbose: bool = False,
          ranks=None) -> dict:
    """Find a patch for (cfg, seed).  Returns the patch dict.

    ``ranks`` ([B, K] ints, -1 = a miss) replaces the ranks drawn from the accuracy
    table, to reach a chosen accepted length; the patch then records them."""
    if isinstance(cfg, str):
        cfg = get_config(cfg)
    log = print if verbose else (lambda *a, **k: None)
    for attempt in range(max_attempts):
        inp = make_inputs(cfg, seed, attempt=attempt)
        if ranks is not None:
            inp.plant_rank = np.asarray(ranks, dtype=np.int32).reshape(cfg.B, cfg.K)
        plan = plan_for(cfg, inp.acc)
        ed = _Editor(inp)
        hf = oracle.as_f64(inp.h, inp.dtype)
        root_lg = oracle.lm_head_logits(inp.w_lm, hf, inp.dtype)
        # root and greedy-chain margins are opened by the lm_head edits below;
        # only an exact tie (no winner to raise) forces a new draw of h
        if min(margin_top1(root_lg[b]) for b in range(cfg.B)) <= 0.0:
            log(f"attempt {attempt}: tied root")
            continue
        root = np.array([oracle.argmax_lowest(root_lg[b]) for b in range(cfg.B)])
        chain, chain_lg = _greedy_chain(inp, plan, root)
        if min(margin_top1(l) for lgs in chain_lg for l in lgs) <= 0.0:
            log(f"attempt {attempt}: tied greedy step")
            continue
        ok = False
        fixes: Dict[tuple, int] = {}
        for it in range(30):
            if not _fix_heads(ed, inp, plan, chain):
                break
            res = oracle.step(inp, plan, root=root)
            # chain and root must be unchanged by the lm_head edits so far
            root2 = np.array([oracle.argmax_lowest(res.root_logits[b]) for b in range(cfg.B)])
            chain2, chain_lg = _greedy_chain(inp, plan, root)
            if not np.array_equal(root2, root) or any(
                    not np.array_equal(a, c) for a, c in zip(chain, chain2)):
                break
            bad = [dc for dc in all_decisions(inp, plan, res, chain_lg) if dc.margin < THR]
            log(f"attempt {attempt} iter {it}: {len(bad)} small margins "
                f"{[(d.kind, d.where, round(d.margin, 4)) for d in bad[:6]]}")
            if not bad:
                ok = True
                break
            for dc in bad:
                if dc.kind == "head":
                    continue            # handled by _fix_heads on the next pass
                b = dc.where[0]
                if dc.kind == "root":
                    x, lg = hf[b], res.root_logits[b]
                elif dc.kind == "chain":
                    _, hid, _ = oracle.greedy_decode(inp, b, int(root[b]), dc.where[1] + 1)
                    x, lg = hid[-1], chain_lg[b][dc.where[1]]
                else:
                    x, lg = res.node_hidden[b, dc.where[1]], res.logits[b, dc.where[1]]
                top2 = oracle.topk(lg, 2)
                # raise the winner; a decision that is still close after that (another
                # decision's fix moved it back) gets its runner-up pushed down as well
                n_fix = fixes.get((dc.kind, dc.where), 0)
                fixes[(dc.kind, dc.where)] = n_fix + 1
                if n_fix % 2 == 0:
                    ed.move("w_lm", -1, int(top2[0]), x, float(lg[top2[1]]) + SPACING)
                else:
                    ed.move("w_lm", -1, int(top2[1]), x, float(lg[top2[0]]) - SPACING)
        if not ok:
            log(f"attempt {attempt}: could not open every margin")
            continue
        patch = {"config": cfg.name, "seed": int(seed), "h_attempt": int(attempt), "thr": THR,
                 "ops": ed.ops}
        if ranks is not None:
            patch["plant_rank"] = inp.plant_rank.tolist()
        # the patch replayed on a fresh draw must give the same bits
        check = make_inputs(cfg, seed, patch=patch)
        for name, arr in inp.tensors().items():
            if not np.array_equal(arr, getattr(check, name)):
                raise AssertionError(f"patch replay differs on {name}")
        alen_expect = [expected_accept_len(plan, inp.plant_rank[b]) for b in range(cfg.B)]
        if list(res.accept_len) != alen_expect:
            log(f"attempt {attempt}: accept {list(res.accept_len)} != planted {alen_expect}")
            continue
        patch["accept_len"] = [int(a) for a in res.accept_len]
        return patch
    raise RuntimeError(f"planting failed for {cfg.name} seed {seed}")


def planted_inputs(cfg, seed: int, **kw):
    """Inputs with a freshly computed plant (small configs; the large ones use
    the stored patches under tests/golden/plants)."""
    return make_inputs(cfg, seed, patch=plant(cfg, seed, **kw))


def save_patch(patch: dict, path: str) -> None:
    with open(path, "w") as f:
        json.dump(patch, f, separators=(",", ":"))
