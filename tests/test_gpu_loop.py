"""GPU parity of the decode loop: rounds of the whole step followed by medusa_advance (the
accepted branch joins the KV cache, its last hidden state and bonus token start the next
round: glossary "Medusa Heads", section "Attention arborescente et acceptation") emit
exactly the plain greedy stream of the oracle ("Medusa Decoding Heads", section "Diepe
duik").  Seeds are chosen so that every greedy decision of the stream has a top-1
margin of at least 2e-2 in fp64; the test asserts it."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import close_node_hidden, close, exact, oracle_plan, planted, say

pytestmark = pytest.mark.gpu

ROUNDS = 4


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from speculative_decoding_amd import lib
    lib()
    return torch.device("cuda:0")


def _gpu_step(inp, dev):
    from speculative_decoding_amd import medusa as M
    from speculative_decoding_amd.step import Dims, MedusaStep, device_weights
    cfg = inp.cfg
    w = device_weights(inp, dev)
    if cfg.tree == "full":
        plan = M.medusa_tree_plan_full(cfg.tree_s)
    else:
        plan = M.medusa_tree_plan_from_accuracy(inp.acc, cfg.tree_s, cfg.n_nodes)
    plan.upload(dev)
    return MedusaStep(Dims.from_config(cfg), w, plan, dev), w


@pytest.mark.parametrize("cfg,seed", [("tiny_loop", 0), ("tiny_loop", 2), ("small_loop", 1),
                                      ("small_loop", 3), ("small_rope_loop", 2),
                                      ("small_rope_loop", 5)])
def test_decode_loop_emits_greedy_stream(dev, cfg, seed):
    import torch
    say(f"[decode loop {cfg} seed {seed}]")
    inp = planted(cfg, seed)
    st, _ = _gpu_step(inp, dev)
    root0, lens, toks, over = st.decode(ROUNDS)
    torch.cuda.synchronize()
    assert int(over.max().item()) == 0, "a branch did not fit in the cache"
    streams = st.streams(lens, toks)
    ref_root0, ref_streams, _ = oracle.decode_loop(inp, oracle_plan(inp), ROUNDS)
    exact("first roots", root0.cpu().numpy(), ref_root0)
    for b in range(inp.cfg.B):
        g, _, lg = oracle.greedy_decode(inp, b, int(ref_root0[b]), len(streams[b]))
        top2 = np.sort(lg, axis=1)[:, -2:]
        assert (top2[:, 1] - top2[:, 0]).min() >= 2e-2, "seed has a near-tie in its greedy stream"
        exact(f"sequence {b} stream", streams[b], g)
        n = min(len(streams[b]), len(ref_streams[b]))
        exact(f"sequence {b} stream vs the oracle loop", streams[b][:n], ref_streams[b][:n])


@pytest.mark.parametrize("cfg,seed", [("small_loop", 3), ("tiny_loop", 0), ("small_rope_loop", 1)])
def test_advance_matches_oracle(dev, cfg, seed):
    import torch
    say(f"[advance {cfg} seed {seed}]")
    inp = planted(cfg, seed)
    st, w = _gpu_step(inp, dev)
    k0 = w["k_cache"].clone()
    st.run(bootstrap_root=True)
    k_tree = st.k_tree.clone()
    nh = st.node_hidden.clone()
    o_dev = st.o.float().cpu().numpy()
    over = torch.full((inp.cfg.B,), -1, dtype=torch.int32, device=dev)
    st.advance(overflow=over)
    torch.cuda.synchronize()
    res = oracle.step(inp, oracle_plan(inp))
    nxt, roots = oracle.advance(inp, oracle_plan(inp), res)
    exact("overflow", over.cpu().numpy(), np.zeros(inp.cfg.B))
    exact("prefix_lens", w["prefix_lens"].cpu().numpy(), nxt.prefix_lens)
    exact("next roots", st.root_ids.cpu().numpy(), roots)
    kc = w["k_cache"]
    for b in range(inp.cfg.B):
        L, a = int(inp.prefix_lens[b]), int(res.accept_len[b])
        path = [int(i) for i in res.accept_nodes[b, : a + 1]]
        # the appended rows are the step's own tree rows, bit for bit
        assert torch.equal(kc[b, L: L + a + 1], k_tree[b, path])
        # everything else in the cache is untouched
        assert torch.equal(kc[b, :L], k0[b, :L]) and torch.equal(kc[b, L + a + 1:], k0[b, L + a + 1:])
        assert torch.equal(w["h"][b], nh[b, path[a]])
        # and they equal the oracle's rows within the activation tolerance
        close(f"seq {b} appended k", kc[b, L: L + a + 1].float().cpu().numpy(),
              oracle.as_f64(nxt.k_cache[b, L: L + a + 1], inp.dtype))
        i_star = path[a]
        close_node_hidden(f"seq {b} next h", w["h"][b].float().cpu().numpy(),
                          oracle.as_f64(nxt.h[b], inp.dtype), o_dev[b, i_star], res.o[b, i_star],
                          res.x[b, i_star], inp.wo, inp.dtype)


def test_advance_overflow_changes_nothing(dev):
    import torch
    say("[advance overflow]")
    inp = planted("tiny", 0)              # the cache is full: L == Lcap
    st, w = _gpu_step(inp, dev)
    st.run(bootstrap_root=True)
    before = {k: w[k].clone() for k in ("k_cache", "v_cache", "prefix_lens", "h")}
    root = st.root_ids.clone()
    over = torch.zeros(1, dtype=torch.int32, device=dev)
    st.advance(overflow=over)
    torch.cuda.synchronize()
    assert int(over.item()) == 1
    for k, v in before.items():
        assert torch.equal(w[k], v), f"{k} changed"
    assert torch.equal(st.root_ids, root)


def test_root_only_loop_is_greedy_decoding(dev):
    """With a root-only tree every round verifies one token and emits one: the loop is plain
    greedy decoding, token for token, run through the same kernels."""
    import torch
    from speculative_decoding_amd import medusa as M
    from speculative_decoding_amd.step import Dims, MedusaStep, device_weights
    say("[decode loop, root-only tree]")
    rounds = 6
    inp = planted("small_loop", 1)
    plan = M.medusa_tree_plan_from_accuracy(inp.acc, inp.cfg.tree_s, 1).upload(dev)
    st = MedusaStep(Dims.from_config(inp.cfg), device_weights(inp, dev), plan, dev)
    root0, lens, toks, over = st.decode(rounds)
    torch.cuda.synchronize()
    assert int(over.max().item()) == 0 and int(lens.max().item()) == 0
    streams = st.streams(lens, toks)
    for b in range(inp.cfg.B):
        g, _, lg = oracle.greedy_decode(inp, b, int(root0[b].item()), rounds)
        top2 = np.sort(lg, axis=1)[:, -2:]
        assert (top2[:, 1] - top2[:, 0]).min() >= 2e-2, "seed has a near-tie in its greedy stream"
        exact(f"sequence {b} stream", streams[b], g)


def test_loop_resumes_from_saved_state(dev, tmp_path):
    """Save the loop state after two rounds (safetensors), finish the loop, then restore the
    state into a fresh step over the original inputs: the remaining rounds emit the same
    tokens."""
    import torch
    say("[decode loop, save and resume]")
    inp = planted("small_loop", 3)
    st, _ = _gpu_step(inp, dev)
    st.decode(2)
    torch.cuda.synchronize()
    path = str(tmp_path / "loop_state.safetensors")
    st.save_loop_state(path)
    _, lens, toks, _ = st.decode(3, bootstrap_root=False)
    torch.cuda.synchronize()
    want = st.streams(lens, toks)

    fresh, _ = _gpu_step(inp, dev)
    fresh.restore_loop_state(path)
    _, lens2, toks2, _ = fresh.decode(3, bootstrap_root=False)
    torch.cuda.synchronize()
    got = fresh.streams(lens2, toks2)
    for b in range(inp.cfg.B):
        exact(f"sequence {b} resumed stream", got[b], want[b])
