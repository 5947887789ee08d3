"""Helpers for the GPU parity tests: run the HIP step and compare with the oracle."""
from __future__ import annotations

import os
import sys
import time

import numpy as np

import oracle
from synth import get_config, make_inputs
from tests import planting

HERE = os.path.dirname(os.path.abspath(__file__))
PLANTS = os.path.join(HERE, "golden", "plants")

RTOL = 2e-2
ATOL = 1e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def close(name: str, got, want, rtol: float = RTOL, atol: float = ATOL,
          row_scale: bool = False) -> None:
    """|gpu - oracle| <= atol + rtol * ref elementwise, with ref = |oracle|, or for a dot
    product output (row_scale) ref = max(|oracle|, RMS of the oracle's last-axis row): an
    output that cancels to near zero carries the same absolute rounding error as the rest
    of its row."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    ref = np.abs(want)
    if row_scale and want.size:
        rms = np.sqrt(np.mean(want * want, axis=-1, keepdims=True))
        ref = np.maximum(ref, rms)
    excess = np.abs(got - want) - (atol + rtol * ref)
    if excess.size and excess.max() > 0:
        i = np.unravel_index(int(np.argmax(excess)), excess.shape)
        raise AssertionError(f"{name}: |gpu-oracle| exceeds {atol}+{rtol}*ref at {i}: "
                             f"gpu {got[i]} oracle {want[i]} "
                             f"({int((excess > 0).sum())} of {excess.size} elements)")


def exact(name: str, got, want) -> None:
    got = np.asarray(got, dtype=np.int64)
    want = np.asarray(want, dtype=np.int64)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError(f"{name}: {len(bad)} mismatches, first at {i}: gpu {got[i]} "
                             f"oracle {want[i]}")


def planted(cfg_name: str, seed: int):
    """Planted inputs: the stored patch when there is one, else a fresh plant."""
    path = os.path.join(PLANTS, f"{cfg_name}_s{seed}.json")
    if os.path.exists(path):
        return make_inputs(cfg_name, seed, patch=path)
    return planting.planted_inputs(cfg_name, seed)


def oracle_plan(inp):
    return planting.plan_for(inp.cfg, inp.acc)


def gpu_plan(inp, device):
    from speculative_decoding_amd import medusa as M
    cfg = inp.cfg
    if cfg.tree == "full":
        p = M.medusa_tree_plan_full(cfg.tree_s)
    else:
        p = M.medusa_tree_plan_from_accuracy(inp.acc, cfg.tree_s, cfg.n_nodes)
    return p.upload(device)


def run_gpu(inp, device, keep_logits=True, bootstrap_root=True, root=None, keep_u=True,
            plan=None, typical=None):
    import torch
    from speculative_decoding_amd.step import Dims, MedusaStep, device_weights
    plan = gpu_plan(inp, device) if plan is None else plan.upload(device)
    step = MedusaStep(Dims.from_config(inp.cfg), device_weights(inp, device), plan, device,
                      keep_logits=keep_logits, typical=typical)
    if root is not None:
        step.root_ids.copy_(torch.as_tensor(np.asarray(root, np.int32), device=device))
    step.run(bootstrap_root=bootstrap_root, keep_u=keep_u)
    torch.cuda.synchronize()
    return step, step.results()


def node_argmax_valid(got_am, ref: "oracle.StepResult", rtol: float = RTOL,
                      atol: float = ATOL) -> int:
    """Node argmax where the verify logits may hold near-ties (nodes the planting did not
    reach): where the GPU differs from the oracle, the oracle's logit of the GPU's token
    must lie within the logits' tolerance of the oracle's maximum (scale: the row's RMS).
    Returns how many nodes took the other side of a near-tie."""
    got_am = np.asarray(got_am, dtype=np.int64)
    assert got_am.shape == ref.node_argmax.shape
    flips = 0
    for b, i in np.argwhere(got_am != ref.node_argmax):
        row = ref.logits[b, i]
        rms = float(np.sqrt(np.mean(row * row)))
        gap = float(row[ref.node_argmax[b, i]] - row[got_am[b, i]])
        lim = atol + rtol * max(abs(float(row[ref.node_argmax[b, i]])), rms)
        assert gap <= lim, (f"node_argmax[{b},{i}]: gpu {got_am[b, i]} is {gap} below the "
                            f"oracle's best {ref.node_argmax[b, i]} (tolerance {lim})")
        flips += 1
    return flips


def compare_step(inp, got: dict, ref: "oracle.StepResult", check_logits: bool = True,
                 check_u: bool = True, plan=None) -> None:
    """Every output of the GPU step against the oracle; reports all mismatches at once.
    Ids, tokens and accept results bit-exact; floating outputs within tolerance.

    With ``plan`` (an oracle plan whose nodes the inputs were not planted for) the node
    argmax may take the other side of a near-tie (``node_argmax_valid``), and the accept
    results must be exactly what the oracle's acceptance rule makes of the GPU's own
    node tokens and argmax; where no node flipped they equal the oracle's."""
    cfg = inp.cfg
    if plan is None:
        decisions = [
            lambda: exact("node_argmax", got["node_argmax"], ref.node_argmax),
            lambda: exact("accept_len", got["accept_len"], ref.accept_len),
            lambda: exact("accept_nodes", got["accept_nodes"], ref.accept_nodes),
            lambda: exact("accept_tokens", got["accept_tokens"], ref.accept_tokens),
        ]
    else:
        def accept_from_gpu_decisions():
            node_argmax_valid(got["node_argmax"], ref)
            alen, anodes, atoks = oracle.accept(plan, got["node_tokens"], got["node_argmax"])
            exact("accept_len", got["accept_len"], alen)
            exact("accept_nodes", got["accept_nodes"], anodes)
            exact("accept_tokens", got["accept_tokens"], atoks)
        decisions = [accept_from_gpu_decisions]
    checks = [
        lambda: exact("root_ids", got["root_ids"], ref.root),
        lambda: exact("topk_ids", got["topk_ids"], ref.topk_ids),
        lambda: exact("node_tokens", got["node_tokens"], ref.tokens),
        lambda: exact("position_ids", got["position_ids"], ref.pos),
    ] + decisions + [
        lambda: close("q", got["q"], ref.q),
        lambda: close("k_tree", got["k_tree"], ref.k),
        lambda: close("v_tree", got["v_tree"], ref.v),
        lambda: close("o", got["o"], ref.o),
        lambda: close("node_hidden", got["node_hidden"], ref.node_hidden),
    ]
    if check_u:
        checks.append(lambda: close("u", got["u"], ref.u))
    for k in range(cfg.K):
        sk = cfg.s[k]
        checks.append(lambda k=k, sk=sk: close(f"topk_vals[head {k}]", got["topk_vals"][:, k, :sk],
                                               ref.topk_vals[:, k, :sk]))
    if check_logits and got.get("head_logits") is not None:
        checks.append(lambda: close("head_logits", got["head_logits"][:, : cfg.K], ref.head_logits,
                                    row_scale=True))
        checks.append(lambda: close("root_logits", got["head_logits"][:, cfg.K], ref.root_logits,
                                    row_scale=True))
    if check_logits and got.get("verify_logits") is not None:
        checks.append(lambda: close("verify_logits", got["verify_logits"], ref.logits,
                                    row_scale=True))
    errors = []
    for c in checks:
        try:
            c()
        except AssertionError as e:
            errors.append(str(e))
    if errors:
        raise AssertionError(f"{cfg.name} seed {inp.seed}: " + "\n".join(errors))
