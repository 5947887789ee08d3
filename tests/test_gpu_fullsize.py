"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times: every id, token and accept result bit-exact, and the verifier's q/k/v, attention
output and node hidden states within tolerance, against the oracle run on the same
planted draw.  Seed 0 of every workload also writes the optional logits (the heads'
and the root's, and every tree node's verification logits; the same kernels, with the
store turned on) and compares them element by element.

Seeds 0-4 (0-2) carry ranks drawn from the accuracy table; the further seeds were
planted for chosen accepted lengths, so that every length 0..D occurs at every shape,
full-depth acceptance (the bonus token from a leaf's argmax) included."""
import os

import numpy as np
import pytest

import oracle
from tests.gpu_util import PLANTS, compare_step, oracle_plan, planted, run_gpu, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

# seeds with a stored plant: 8B and Mid 0-4, Dense and Batched 70B 0-2 (drawn ranks);
# 8B 7-8 (accept 3, 4), Mid 5-7 (0, 4, 5), Dense 3-5 (1, 2, 4) with chosen ranks
CASES = ([("8b", s) for s in (0, 1, 2, 3, 4, 7, 8)] + [("mid", s) for s in range(8)] +
         [("dense", s) for s in range(6)] + [("batched70b", s) for s in range(3)])


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from speculative_decoding_amd import lib
    lib()
    return torch.device("cuda:0")


@pytest.mark.parametrize("cfg,seed", CASES)
def test_full_size_step(dev, cfg, seed):
    import torch
    path = os.path.join(PLANTS, f"{cfg}_s{seed}.json")
    if not os.path.exists(path):
        pytest.skip(f"no stored plant for {cfg} seed {seed}")
    say(f"[full size {cfg} seed {seed}] generating")
    inp = planted(cfg, seed)
    with_logits = seed == 0
    say(f"[full size {cfg} seed {seed}] gpu step (logits {with_logits})")
    step, got = run_gpu(inp, dev, keep_logits=with_logits, keep_u=False)
    del step
    torch.cuda.empty_cache()
    say(f"[full size {cfg} seed {seed}] oracle step")
    ref = oracle.step(inp, oracle_plan(inp))
    compare_step(inp, got, ref, check_logits=with_logits, check_u=False)
    want = inp.patch.get("accept_len")
    if want is not None:
        assert got["accept_len"].tolist() == want, (got["accept_len"].tolist(), want)
    say(f"[full size {cfg} seed {seed}] accept {got['accept_len'].tolist()}")
