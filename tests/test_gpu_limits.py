"""GPU parity at the library's limits, at small shapes: eight heads (the most allowed),
top-64 on the first (the largest top-k), and a 1024-node tree (the largest plan: depth 8,
sixteen mask words, 2048 verified rows over two sequences) with an empty and a ragged
prefix; and the largest batch, 64 sequences.  The inputs are not planted (planting opens
no margins at 2048 nodes, nor across 64 sequences sharing the heads), so each
node's argmax may take either side of a near-tie and the accept results must follow from
the device's own decisions; the heads' top-65 gaps are checked to be far above the fp32
rounding of the device's logits, so their top-k is exact."""
import numpy as np
import pytest

import oracle
from synth import make_inputs
from tests.gpu_util import compare_step, oracle_plan, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from speculative_decoding_amd import lib
    lib()
    return torch.device("cuda:0")


def test_limits_step(dev):
    say("[limits: K=8, top-64, 1024 nodes, B=2]")
    inp = make_inputs("small_max", 0)
    cfg = inp.cfg
    plan = oracle_plan(inp)
    assert plan.n_nodes == 1024 and plan.max_depth == 8 and plan.mask_words == 16
    ref = oracle.step(inp, plan)
    for b in range(cfg.B):
        for k in range(cfg.K):
            v = np.sort(ref.head_logits[b, k])[::-1][: cfg.s[k] + 1]
            assert np.min(v[:-1] - v[1:]) >= 1e-4, "the draw has a near-tie in a head's top-k"
    _, got = run_gpu(inp, dev, keep_logits=False, keep_u=False)
    compare_step(inp, got, ref, plan=plan, check_logits=False, check_u=False)
    say(f"    accept {got['accept_len'].tolist()}")


def test_batch64_step(dev):
    """The largest batch the heads accept: 64 sequences (row-streaming heads over four
    16-row blocks, 576 verified rows), prefixes from empty to the full cache."""
    say("[limits: B=64]")
    inp = make_inputs("small_b64", 2)
    cfg = inp.cfg
    assert int(inp.prefix_lens.min()) == 0 and int(inp.prefix_lens.max()) == cfg.Lcap
    plan = oracle_plan(inp)
    ref = oracle.step(inp, plan)
    for b in range(cfg.B):
        r = np.sort(ref.root_logits[b])[-2:]
        assert r[1] - r[0] >= 1e-4, "the draw has a near-tie at a root"
        for k in range(cfg.K):
            v = np.sort(ref.head_logits[b, k])[::-1][: cfg.s[k] + 1]
            assert np.min(v[:-1] - v[1:]) >= 1e-4, "the draw has a near-tie in a head's top-k"
    _, got = run_gpu(inp, dev, keep_logits=True)
    compare_step(inp, got, ref, plan=plan)
    say(f"    accept {got['accept_len'].tolist()}")


@pytest.mark.parametrize("V", [65535, 65536])
def test_vocabulary_tile_boundary(dev, V):
    """Verification at up to 64 rows takes 64-row vocabulary tiles below 65536 rows and
    256-row tiles from there: a whole step on each side of the switch (the small shape with
    its vocabulary widened), unplanted, so accept results follow the device's decisions."""
    import dataclasses
    from synth import get_config
    say(f"[limits: vocabulary {V}]")
    cfg = dataclasses.replace(get_config("small"), name=f"small_v{V}", V=V)
    inp = make_inputs(cfg, 0)
    plan = oracle_plan(inp)
    ref = oracle.step(inp, plan)
    r = np.sort(ref.root_logits[0])[-2:]
    assert r[1] - r[0] >= 1e-4, "the draw has a near-tie at the root"
    for k in range(cfg.K):
        v = np.sort(ref.head_logits[0, k])[::-1][: cfg.s[k] + 1]
        assert np.min(v[:-1] - v[1:]) >= 1e-4, "the draw has a near-tie in a head's top-k"
    _, got = run_gpu(inp, dev, keep_logits=True)
    compare_step(inp, got, ref, plan=plan)


@pytest.mark.parametrize("base", ["small", "small_batched"])
def test_contraction_off_256(dev, base):
    """Verification over a small vocabulary, and the heads from batch 3, stream 256-wide
    contraction chunks when 256 divides the hidden size and 64-wide chunks otherwise: a
    whole step with H = 448 (a multiple of 64, not of 256) at one sequence and at three,
    unplanted, so accept results follow the device's decisions."""
    import dataclasses
    from synth import get_config
    say(f"[limits: {base}, hidden 448]")
    cfg = dataclasses.replace(get_config(base), name=f"{base}_h448", H=448)
    inp = make_inputs(cfg, 0)
    plan = oracle_plan(inp)
    ref = oracle.step(inp, plan)
    for b in range(cfg.B):
        r = np.sort(ref.root_logits[b])[-2:]
        assert r[1] - r[0] >= 1e-4, "the draw has a near-tie at a root"
        for k in range(cfg.K):
            v = np.sort(ref.head_logits[b, k])[::-1][: cfg.s[k] + 1]
            assert np.min(v[:-1] - v[1:]) >= 1e-4, "the draw has a near-tie in a head's top-k"
    _, got = run_gpu(inp, dev, keep_logits=True)
    compare_step(inp, got, ref, plan=plan)
    say(f"    accept {got['accept_len'].tolist()}")


@pytest.mark.parametrize("B", [1, 2])
def test_small_vocabulary_row_blocks(dev, B):
    """Verification over a small vocabulary takes 16-, 32- or 64-row input blocks: the
    small batched shape (16-node trees) at one and two sequences verifies 16 and 32 rows,
    unplanted, so accept results follow the device's decisions."""
    import dataclasses
    from synth import get_config
    say(f"[limits: small_batched, B={B}]")
    base = get_config("small_batched")
    cfg = dataclasses.replace(base, name=f"small_batched_b{B}", B=B, lens=base.lens[:B])
    inp = make_inputs(cfg, 0)
    plan = oracle_plan(inp)
    ref = oracle.step(inp, plan)
    for b in range(cfg.B):
        r = np.sort(ref.root_logits[b])[-2:]
        assert r[1] - r[0] >= 1e-4, "the draw has a near-tie at a root"
        for k in range(cfg.K):
            v = np.sort(ref.head_logits[b, k])[::-1][: cfg.s[k] + 1]
            assert np.min(v[:-1] - v[1:]) >= 1e-4, "the draw has a near-tie in a head's top-k"
    _, got = run_gpu(inp, dev, keep_logits=True)
    compare_step(inp, got, ref, plan=plan)
    say(f"    accept {got['accept_len'].tolist()}")
