"""GPU parity of typical acceptance (medusa_verify_accept_typical) against the oracle's
typical_accept, on planted inputs (every node's argmax has a margin, so node tokens and
argmax are exact).  Each candidate's probability under its parent's distribution and each
node's threshold are fp32 on the device and within tolerance of the oracle's fp64; the
accept results must be exactly what the walk makes of the device's own probabilities and
thresholds, and equal the oracle's wherever no decision on the way sits within the
tolerance of its threshold.  At a temperature near zero the result is greedy acceptance
bit for bit."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import (close, close_node_hidden, close_verify_logits, exact, oracle_plan,
                            planted, run_gpu, say)

pytestmark = pytest.mark.gpu

PROB_RTOL = 2e-2
PROB_ATOL = 1e-30

# (config, seed, temperature, epsilon, delta, sure); configurations cover the fp32 kernel
# (tiny), the row-streaming kernel with one 64-row block (small), with 128-row blocks past
# 64 verified rows (small_dense: 170 rows over two sequences; small_n341), several sequences
# (small_batched, small_dense), flat (T = 1) and sharp (small T) distributions.  Where
# ``sure`` is set the oracle puts no candidate within tolerance of its threshold (checked
# in the test), so the accept results must equal the oracle's.
CASES = [
    ("tiny", 0, 1.0, 0.3, 0.09, True),
    ("tiny", 2, 0.2, 0.09, 0.3, True),
    ("small", 0, 1.0, 0.09, 0.3, True),
    ("small", 1, 0.05, 0.09, 0.3, True),
    ("small_batched", 0, 0.5, 0.2, 0.5, True),
    ("small_dense", 0, 1.0, 0.09, 0.3, False),
    ("small_dense", 0, 0.7, 0.05, 0.5, True),
    ("small_n341", 0, 0.7, 0.05, 0.5, False),
    ("small_n341", 0, 0.5, 0.09, 0.3, True),
]


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from speculative_decoding_amd import lib
    lib()
    return torch.device("cuda:0")


def _close_calls(plan, prob, tau):
    """Candidates whose probability sits within the tolerance of their parent's threshold."""
    B, N = prob.shape
    n = 0
    for bb in range(B):
        for i in range(1, N):
            par = int(plan.parent[i])
            if abs(prob[bb, i] - tau[bb, par]) <= PROB_RTOL * max(prob[bb, i], tau[bb, par]):
                n += 1
    return n


def _check_typical(inp, got, ref, plan, T, eps, delta, sure=False):
    """Typical acceptance, stage by stage: the node hidden states against the oracle (with
    the flip term of their bf16 input o); the probabilities and thresholds against the
    oracle's rule applied to the oracle's lm_head of the device's own node hidden states
    (lm_head itself is checked in the step tests); the accept results against the device's
    own walk, and against the oracle's decisions when none sits within tolerance of its
    threshold."""
    a, nodes, toks, prob, tau = oracle.typical_accept(plan, ref.tokens, ref.logits,
                                                      ref.node_argmax, T, eps, delta)
    exact("root_ids", got["root_ids"], ref.root)
    exact("node_tokens", got["node_tokens"], ref.tokens)
    exact("node_argmax", got["node_argmax"], ref.node_argmax)
    close_node_hidden("node_hidden", got["node_hidden"], ref.node_hidden, got["o"], ref.o, ref.x,
                      inp.wo, inp.dtype)
    own_logits = oracle.verify(np.asarray(got["node_hidden"], np.float64), inp.w_lm, inp.dtype)[0]
    a_own, nodes_own, toks_own, prob_own, tau_own = oracle.typical_accept(
        plan, ref.tokens, own_logits, ref.node_argmax, T, eps, delta)
    close("node_prob", got["node_prob"], prob_own, rtol=PROB_RTOL, atol=PROB_ATOL)
    close("node_tau", got["node_tau"], tau_own, rtol=PROB_RTOL, atol=PROB_ATOL)
    # the device's walk over its own probabilities and thresholds
    ga, gn, gt = oracle.typical_branch(plan, got["node_tokens"], got["node_argmax"],
                                       got["node_prob"].astype(np.float64),
                                       got["node_tau"].astype(np.float64))
    exact("accept_len (device rule)", got["accept_len"], ga)
    exact("accept_nodes (device rule)", got["accept_nodes"], gn)
    exact("accept_tokens (device rule)", got["accept_tokens"], gt)
    # and the oracle's decisions, on both sets of logits, where none is within tolerance
    close_calls = _close_calls(plan, prob, tau) + _close_calls(plan, prob_own, tau_own)
    if sure:
        assert close_calls == 0, f"{close_calls} oracle decisions sit within tolerance"
    if close_calls == 0:
        for name, g, o1, o2 in (("accept_len", got["accept_len"], a, a_own),
                                ("accept_nodes", got["accept_nodes"], nodes, nodes_own),
                                ("accept_tokens", got["accept_tokens"], toks, toks_own)):
            exact(name, g, o1)
            exact(name + " (oracle on the device's node_hidden)", g, o2)
    say(f"    accept {got['accept_len'].tolist()} (oracle {a.tolist()}), "
        f"{close_calls} decisions within tolerance of the threshold")


@pytest.mark.parametrize("cfg,seed,T,eps,delta,sure", CASES)
def test_typical_step(dev, cfg, seed, T, eps, delta, sure):
    say(f"[typical {cfg} seed {seed} T={T} eps={eps} delta={delta}]")
    inp = planted(cfg, seed)
    plan = oracle_plan(inp)
    ref = oracle.step(inp, plan)
    _, got = run_gpu(inp, dev, typical=(T, eps, delta))
    _check_typical(inp, got, ref, plan, T, eps, delta, sure)
    close_verify_logits("verify_logits", got["verify_logits"], ref.logits, got["node_hidden"],
                        ref.node_hidden, inp.w_lm, inp.dtype)


@pytest.mark.parametrize("cfg,seed", [("tiny", 1), ("small", 0), ("small_batched", 1),
                                      ("small_dense", 1)])
def test_typical_low_temperature_is_greedy(dev, cfg, seed):
    """T = 1e-4 with planted margins >= 1e-2: only the argmax keeps any probability, so
    typical acceptance makes exactly the greedy decisions."""
    say(f"[typical T=1e-4 {cfg} seed {seed}]")
    inp = planted(cfg, seed)
    _, greedy = run_gpu(inp, dev, keep_logits=False)
    _, typ = run_gpu(inp, dev, keep_logits=False, typical=(1e-4, 0.09, 0.3))
    for name in ("node_argmax", "accept_len", "accept_nodes", "accept_tokens"):
        exact(name, typ[name], greedy[name])
    assert set(np.unique(typ["node_prob"]).tolist()) <= {0.0, 1.0} or \
        np.all((typ["node_prob"] < 1e-30) | (typ["node_prob"] > 1 - 1e-6))


def test_typical_run_twice_bitwise(dev):
    import torch
    inp = planted("small_dense", 0)
    step, first = run_gpu(inp, dev, keep_logits=False, typical=(0.7, 0.09, 0.3))
    step.run(bootstrap_root=True)
    torch.cuda.synchronize()
    second = step.results()
    for name in ("node_prob", "node_tau"):
        assert np.array_equal(first[name].view(np.uint32), second[name].view(np.uint32)), name
    for name in ("accept_len", "accept_nodes", "accept_tokens", "node_argmax"):
        exact(name, second[name], first[name])


@pytest.mark.slow
@pytest.mark.parametrize("cfg", ["8b", "mid"])
def test_typical_full_size(dev, cfg):
    """The benchmark shapes: 8B (256-row vocabulary tiles) and 7B (vocabulary 32000,
    64-row tiles)."""
    import os
    import torch
    from tests.gpu_util import PLANTS
    if not os.path.exists(os.path.join(PLANTS, f"{cfg}_s0.json")):
        pytest.skip(f"no stored plant for {cfg} seed 0")
    say(f"[typical {cfg} seed 0] generating")
    inp = planted(cfg, 0)
    plan = oracle_plan(inp)
    say(f"[typical {cfg} seed 0] gpu step")
    step, got = run_gpu(inp, dev, keep_logits=False, keep_u=False, typical=(0.5, 0.09, 0.3))
    del step
    torch.cuda.empty_cache()
    say(f"[typical {cfg} seed 0] oracle step")
    ref = oracle.step(inp, plan)
    _check_typical(inp, got, ref, plan, 0.5, 0.09, 0.3)
