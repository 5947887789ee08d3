"""GPU parity of the step across tree budgets: the same planted inputs verified through
sparse trees of other sizes than the one they were planted for (the root alone, a few
nodes, several 64-row blocks of verified rows with a ragged last one), at the small parity
shape and at the 8B shape.  Nodes outside the planted tree have no guaranteed margin, so
their argmax may take the other side of a near-tie; everything else is exact or within
tolerance as in the other parity tests, and the accept results must follow from the GPU's
own decisions by the oracle's rule."""
import os

import pytest

import oracle
from tests.gpu_util import PLANTS, compare_step, planted, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from speculative_decoding_amd import lib
    lib()
    return torch.device("cuda:0")


def _budget_case(dev, cfg_name, seed, n, **kw):
    from speculative_decoding_amd import medusa as M
    inp = planted(cfg_name, seed)
    cfg = inp.cfg
    oplan = oracle.plan_from_accuracy(inp.acc, cfg.tree_s, n)
    gplan = M.medusa_tree_plan_from_accuracy(inp.acc, cfg.tree_s, n)
    say(f"[budget {cfg_name} seed {seed} nodes {n}] gpu step")
    step, got = run_gpu(inp, dev, plan=gplan, **kw)
    del step
    say(f"[budget {cfg_name} seed {seed} nodes {n}] oracle step")
    ref = oracle.step(inp, oplan)
    compare_step(inp, got, ref, plan=oplan, check_logits=kw.get("keep_logits", True),
                 check_u=kw.get("keep_u", True))
    say(f"[budget {cfg_name} seed {seed} nodes {n}] accept {got['accept_len'].tolist()}")


@pytest.mark.parametrize("n", [1, 2, 33, 128, 341])
def test_small_budget(dev, n):
    _budget_case(dev, "small", 0, n)


@pytest.mark.slow
@pytest.mark.parametrize("n", [1, 341])
def test_8b_budget(dev, n):
    import torch
    if not os.path.exists(os.path.join(PLANTS, "8b_s0.json")):
        pytest.skip("no stored plant for 8b seed 0")
    _budget_case(dev, "8b", 0, n, keep_logits=False, keep_u=False)
    torch.cuda.empty_cache()
