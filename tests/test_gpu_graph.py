"""The step and the decode loop captured in a graph: the library's calls enqueue kernels
only (no allocation, no memset, no synchronisation), so a caller may capture them.  Every
replay, with eager work and synchronisations between replays, must give the eager
results bit for bit."""
import numpy as np
import pytest

from tests.gpu_util import exact, planted, say

pytestmark = pytest.mark.gpu

OUTS = ("node_tokens", "node_argmax", "accept_len", "accept_nodes", "accept_tokens")


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from speculative_decoding_amd import lib
    lib()
    return torch.device("cuda:0")


def _step(inp, dev, **kw):
    from speculative_decoding_amd import medusa as M
    from speculative_decoding_amd.step import Dims, MedusaStep, device_weights
    cfg = inp.cfg
    if cfg.tree == "full":
        plan = M.medusa_tree_plan_full(cfg.tree_s)
    else:
        plan = M.medusa_tree_plan_from_accuracy(inp.acc, cfg.tree_s, cfg.n_nodes)
    plan.upload(dev)
    return MedusaStep(Dims.from_config(cfg), device_weights(inp, dev), plan, dev, **kw)


@pytest.mark.parametrize("cfg,typical", [("small_batched", None), ("small_dense", None),
                                         ("small", (0.7, 0.09, 0.3))])
def test_step_graph_replays(dev, cfg, typical):
    import torch
    say(f"[graph step {cfg} typical={typical}]")
    inp = planted(cfg, 0)
    st = _step(inp, dev, typical=typical)
    st.run(bootstrap_root=True)          # eager: bootstrap root, one-time launch set-up
    torch.cuda.synchronize()
    want = {k: getattr(st, k).clone() for k in OUTS + ("node_hidden", "o")}
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            st.run(bootstrap_root=False, keep_u=False)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for r in range(3):
        for k in OUTS:                   # eager work between replays: clear the outputs
            getattr(st, k).fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in want.items():
            assert torch.equal(getattr(st, k), v), f"replay {r}: {k} differs from the eager step"


def test_loop_graph_matches_eager_loop(dev):
    """One round (step + advance) captured once and replayed: the rounds continue from the
    state the previous replay left, and emit the eager loop's tokens."""
    import torch
    say("[graph loop small_loop seed 3]")
    rounds = 4
    inp = planted("small_loop", 3)
    eager = _step(inp, dev)
    _, lens, toks, over = eager.decode(rounds)
    torch.cuda.synchronize()
    want = eager.streams(lens, toks)

    st = _step(inp, dev)
    st.run(bootstrap_root=True, keep_u=False)            # round 0 eagerly (bootstrap root)
    got_lens, got_toks = [st.accept_len.cpu()], [st.accept_tokens.cpu()]
    st.advance()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            st.run(bootstrap_root=False, keep_u=False)
            st.advance()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    # capturing recorded the round without running it: replay rounds 1 .. rounds-1
    for _ in range(rounds - 1):
        g.replay()
        torch.cuda.synchronize()
        got_lens.append(st.accept_len.cpu())
        got_toks.append(st.accept_tokens.cpu())
    got = st.streams(torch.stack(got_lens), torch.stack(got_toks))
    for b in range(inp.cfg.B):
        exact(f"sequence {b} stream", np.asarray(got[b]), np.asarray(want[b]))
