"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times (no optional logits or head-hidden outputs): every id, token and accept result
bit-exact, and the verifier's q/k/v, attention output and node hidden states within
tolerance, against the oracle run on the same planted draw."""
import os

import numpy as np
import pytest

import oracle
from tests.gpu_util import PLANTS, compare_step, oracle_plan, planted, run_gpu, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

# seeds with a stored plant: 8B and Mid 0-4, Dense and Batched 70B 0-2
CASES = ([("8b", s) for s in range(5)] + [("mid", s) for s in range(5)] +
         [("dense", s) for s in range(3)] + [("batched70b", s) for s in range(3)])


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
    say(f"[full size {cfg} seed {seed}] gpu step")
    step, got = run_gpu(inp, dev, keep_logits=False, keep_u=False)
    del step
    torch.cuda.empty_cache()
    say(f"[full size {cfg} seed {seed}] oracle step")
    ref = oracle.step(inp, oracle_plan(inp))
    compare_step(inp, got, ref, check_logits=False, check_u=False)
    say(f"[full size {cfg} seed {seed}] accept {got['accept_len'].tolist()}")
