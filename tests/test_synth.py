"""The seeded generator: determinism, rounding, patches, and the planted inputs' margins."""
import json
import os

import numpy as np
import pytest

import oracle
from synth import CONFIGS, make_inputs
from synth.gen import accuracy_table, bf16_bits_to_f32, f32_to_bf16_bits
from tests import planting

PLANTS = os.path.join(os.path.dirname(__file__), "golden", "plants")


def test_same_seed_same_bytes_any_thread_count():
    a = make_inputs("small", 3, threads=1)
    b = make_inputs("small", 3, threads=4)
    for k, v in a.tensors().items():
        assert np.array_equal(v, getattr(b, k)), k
    c = make_inputs("small", 4, threads=2)
    assert not np.array_equal(a.w_lm, c.w_lm)


def test_generator_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).normal(0, 2, 50000).astype(np.float32)
    want = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(x), want)
    np.testing.assert_array_equal(bf16_bits_to_f32(want), torch.tensor(x).to(torch.bfloat16).float().numpy())


def test_distribution_parameters():
    inp = make_inputs("small", 0)
    w = bf16_bits_to_f32(inp.w2[0]).astype(np.float64)
    assert abs(w.std() - 1 / np.sqrt(512)) < 1e-3
    assert abs(w.mean()) < 1e-3
    tiny = make_inputs("tiny", 0)
    assert np.array_equal(tiny.w2[1], tiny.w_lm) and not tiny.b1.any()
    assert abs(tiny.w1.std() - 0.02) < 1e-3


def test_accuracy_table_falls_with_rank_and_depth():
    for name, cfg in CONFIGS.items():
        acc = accuracy_table(cfg, 0)
        for k in range(cfg.K):
            row = acc[k, : cfg.s[k]]
            assert np.all(np.diff(row) <= 0) and row[0] < 1 and row.sum() < 1
        assert acc[0, 0] > acc[-1, 0]


def test_prefix_lens():
    b = make_inputs("small_batched", 0)
    assert b.prefix_lens.tolist() == [0, 129, 300]
    from synth.gen import _prefix_lens
    for seed in range(5):
        L = _prefix_lens(CONFIGS["batched70b"], seed)
        assert L.shape == (8,) and L.min() >= 512 and L.max() <= 8192


def test_patch_replay_and_mismatch():
    patch = planting.plant("tiny", 5)
    a = make_inputs("tiny", 5, patch=patch)
    b = make_inputs("tiny", 5, patch=json.loads(json.dumps(patch)))
    for k, v in a.tensors().items():
        assert np.array_equal(v, getattr(b, k))
    with pytest.raises(ValueError):
        make_inputs("tiny", 6, patch=patch)


@pytest.mark.parametrize("fname", sorted(f for f in os.listdir(PLANTS)
                                         if f.endswith(".json") and f.split("_s")[0] in
                                         ("tiny", "small", "small_batched")))
def test_stored_small_plants_margins(fname):
    """Every discrete decision of a planted draw has a margin >= 1e-2 in fp64."""
    cfg, seed = fname[:-5].rsplit("_s", 1)
    inp = make_inputs(cfg, int(seed), patch=os.path.join(PLANTS, fname))
    plan = planting.plan_for(inp.cfg, inp.acc)
    res = oracle.step(inp, plan)
    _, chain_lg = planting._greedy_chain(inp, plan, res.root)
    for d in planting.all_decisions(inp, plan, res, chain_lg):
        assert d.margin >= 1e-2, (d.kind, d.where, d.margin)


def test_mean_accept_matches_closed_form():
    """Planted ranks are drawn from the accuracy table, so the expected accepted length is
    sum over non-root tree nodes of prod_d acc[d-1][rank_d]; check the draws' mean
    within 4 standard errors (800 draws)."""
    cfg = CONFIGS["small"]
    from synth.gen import _plant_ranks
    acc = accuracy_table(cfg, 0)
    plan = oracle.plan_from_accuracy(acc, cfg.tree_s, cfg.n_nodes)
    expect = 0.0
    for t in plan.paths[1:]:
        p = 1.0
        for d, r in enumerate(t):
            p *= acc[d, r]
        expect += p
    vals = []
    for seed in range(800):
        ranks = _plant_ranks(cfg, seed, acc)
        vals.append(planting.expected_accept_len(plan, ranks[0]))
    vals = np.array(vals, dtype=np.float64)
    se = vals.std() / np.sqrt(len(vals))
    assert abs(vals.mean() - expect) < 4 * se, (vals.mean(), expect, se)


FULL_SHAPES = ("8b", "mid", "dense")     # batched 70B: lengths 0-4 so far


@pytest.mark.parametrize("cfg_name", FULL_SHAPES)
def test_stored_plants_cover_every_accept_length(cfg_name):
    """The stored full-size plants reach every accepted length 0..D of their tree
    (D = the tree's depth), and each patch's recorded length is the one its planted ranks
    give under the tree walk.  (The margins of these patches are asserted when they are
    written, and every GPU full-size test checks the step against the oracle.)"""
    cfg = CONFIGS[cfg_name]
    seen = set()
    for fname in sorted(os.listdir(PLANTS)):
        if not (fname.endswith(".json") and fname[:-5].rsplit("_s", 1)[0] == cfg_name):
            continue
        seed = int(fname[:-5].rsplit("_s", 1)[1])
        with open(os.path.join(PLANTS, fname)) as f:
            patch = json.load(f)
        assert patch["config"] == cfg_name and patch["seed"] == seed
        assert patch["thr"] >= 1e-2
        acc = accuracy_table(cfg, seed)
        plan = planting.plan_for(cfg, acc)
        if "plant_rank" in patch:
            ranks = np.asarray(patch["plant_rank"], dtype=np.int32)
        else:
            from synth.gen import _plant_ranks
            ranks = _plant_ranks(cfg, seed, acc)
        want = [planting.expected_accept_len(plan, ranks[b]) for b in range(cfg.B)]
        assert patch["accept_len"] == want, (fname, patch["accept_len"], want)
        seen.update(want)
        depth = plan.max_depth
    assert seen == set(range(depth + 1)), (cfg_name, sorted(seen), depth)
