"""medusa_verify_accept_noalloc (verification with the library's static scratch instead of a
caller workspace) against medusa_verify_accept on the same inputs, through the C ABI: node
argmax, accepted lengths, nodes and tokens bit-exact, and the optional logits identical
(the same kernels run in both).  Two calls in a row, the second on a smaller problem (fewer
sequences and a smaller vocabulary) so that it runs over what the first left in the
scratch; and a problem larger than the scratch is refused before anything runs."""
import numpy as np
import pytest

from synth import integers, normal_bf16
from tests.gpu_util import exact, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from speculative_decoding_amd import lib
    lib()
    return torch.device("cuda:0")


def _inputs(dev, seed, B, H, V, plan_n):
    import torch
    from speculative_decoding_amd.step import host_to_device
    hid = normal_bf16(seed, "noalloc.hidden", (B, plan_n, H), 1.0)
    w = normal_bf16(seed, "noalloc.w_lm", (V, H), 1.0 / np.sqrt(H))
    toks = integers(seed, "noalloc.tokens", 0, V, (B, plan_n)).astype(np.int32)
    return (host_to_device(hid, "bf16", dev), host_to_device(w, "bf16", dev),
            torch.as_tensor(toks, device=dev))


def _outputs(dev, B, N, D, V):
    import torch
    i32 = dict(dtype=torch.int32, device=dev)
    return dict(node_argmax=torch.full((B, N), -7, **i32), accept_len=torch.full((B,), -7, **i32),
                accept_nodes=torch.full((B, D + 1), -7, **i32),
                accept_tokens=torch.full((B, D + 1), -7, **i32),
                logits=torch.full((B, N, V), float("nan"), dtype=torch.float32, device=dev))


def _both(dev, plan, B, H, V, seed):
    import torch
    from speculative_decoding_amd import medusa as M
    N, D = plan.n_nodes, plan.max_depth
    hid, w, toks = _inputs(dev, seed, B, H, V, N)
    # plant agreement along a few branches, so the walk accepts candidates: a node's token
    # is its parent's argmax wherever the first pass says so
    ref = _outputs(dev, B, N, D, V)
    ws = torch.empty(M.medusa_verify_workspace(plan, "bf16", B, H, V), dtype=torch.uint8,
                     device=dev)
    M.medusa_verify_accept(plan, "bf16", B, H, V, hid, w, toks, ref["node_argmax"],
                           ref["accept_len"], ref["accept_nodes"], ref["accept_tokens"],
                           ref["logits"], ws)
    torch.cuda.synchronize()
    parent = plan.arrays()[0]
    am = ref["node_argmax"].cpu().numpy()
    t = toks.cpu().numpy()
    for b in range(B):
        for i in range(1, N):
            if (i + b) % 3 != 0:
                t[b, i] = am[b, parent[i]]
    toks = torch.as_tensor(t, device=dev)
    ref = _outputs(dev, B, N, D, V)
    M.medusa_verify_accept(plan, "bf16", B, H, V, hid, w, toks, ref["node_argmax"],
                           ref["accept_len"], ref["accept_nodes"], ref["accept_tokens"],
                           ref["logits"], ws)
    got = _outputs(dev, B, N, D, V)
    M.medusa_verify_accept_noalloc(plan, "bf16", B, H, V, hid, w, toks, got["node_argmax"],
                                   got["accept_len"], got["accept_nodes"], got["accept_tokens"],
                                   got["logits"])
    # and once more without the optional outputs (the node argmax then lives in the scratch)
    bare = _outputs(dev, B, N, D, V)
    M.medusa_verify_accept_noalloc(plan, "bf16", B, H, V, hid, w, toks, None,
                                   bare["accept_len"], bare["accept_nodes"],
                                   bare["accept_tokens"], None)
    torch.cuda.synchronize()
    for name in ("node_argmax", "accept_len", "accept_nodes", "accept_tokens"):
        exact(name, got[name].cpu().numpy(), ref[name].cpu().numpy())
    for name in ("accept_len", "accept_nodes", "accept_tokens"):
        exact(name + " (no optional outputs)", bare[name].cpu().numpy(), ref[name].cpu().numpy())
    a = got["logits"].cpu().numpy()
    r = ref["logits"].cpu().numpy()
    assert np.array_equal(a.view(np.uint32), r.view(np.uint32)), "logits differ"
    return ref["accept_len"].cpu().numpy()


def test_noalloc_equals_workspace_call_twice(dev):
    from speculative_decoding_amd import medusa as M
    acc = np.array([[0.5, 0.2, 0.1], [0.4, 0.2, 0.1], [0.3, 0.2, 0.1]])
    plan = M.medusa_tree_plan_from_accuracy(acc, (3, 3, 3), 16)
    plan.upload(dev)
    say("[noalloc] call 1: 3 sequences, vocabulary 70001")
    a1 = _both(dev, plan, 3, 512, 70001, 0)
    say(f"    accept {a1.tolist()}")
    say("[noalloc] call 2: 1 sequence, vocabulary 5003")
    a2 = _both(dev, plan, 1, 512, 5003, 1)
    say(f"    accept {a2.tolist()}")
    assert max(a1.max(), a2.max()) >= 1


def test_noalloc_refuses_more_than_its_scratch(dev):
    import torch
    from speculative_decoding_amd import medusa as M
    plan = M.medusa_tree_plan_full((4, 4, 4, 4))             # 341 nodes
    plan.upload(dev)
    B, H, V = 16, 4096, 128256
    assert M.medusa_verify_workspace(plan, "bf16", B, H, V) > M.MEDUSA_NOALLOC_SCRATCH_BYTES
    dummy = torch.zeros(16, dtype=torch.int32, device=dev)
    fake = torch.zeros(16, dtype=torch.bfloat16, device=dev)
    with pytest.raises(M.MedusaError) as err:
        M.medusa_verify_accept_noalloc(plan, "bf16", B, H, V, fake, fake, dummy, None, dummy,
                                       dummy, dummy)
    assert err.value.status == 5
