"""GPU parity of tree-masked attention (medusa_tree_attention) on its own, against the
oracle's tree_attention, element by element at 1e-3 + 2e-2 * |oracle| (glossary "Medusa
Heads", section "Attention arborescente et acceptation": each node sees the prefix and its
own ancestors).

The bf16 kernel computes 32 x 32 tiles, one 32-row query tile per wave.  Below 512 query
rows per kv head a workgroup has four waves running in lock step; from 512 on it has eight,
in two groups one phase apart (one group's softmax overlaps the other's matrix products),
with the prefix keys fetched by bounds-checked buffer loads.  The workgroups of a (kv head,
row block) are shared out over the sequences' actual key counts, so the shapes also take
many ragged sequences and trees larger than a chunk.  The shapes cover both schedules, head dims 64 and 128, several query-row blocks with a ragged last one, empty,
short (under one 32-key half) and ragged prefixes, prefixes that end inside a 64-key block
or exactly on one, several prefix splits, multi-head and grouped-query layouts, and the
8B-class shape.  Three cases put values beyond fp16's range (|v| up to 9e4) into the keys'
values: the workgroups that meet them recompute their rows in fp32, and the result must still match."""
import numpy as np
import pytest

import oracle
from synth import integers, normal_bf16
from tests.gpu_util import close, say

pytestmark = pytest.mark.gpu

# name: (B, tree, Hq, Hkv, d, prefix lengths, Lcap, big values)
# tree: ("full", widths) or ("sparse", widths, n_nodes)
CASES = {
    "r1_d128_sparse16": (1, ("sparse", (4, 3, 2), 16), 8, 2, 128, (300,), 320, False),
    "r2_d128_8b_tree": (1, ("sparse", (10, 5, 4, 3), 64), 32, 8, 128, (1000,), 1024, False),
    "r2_d128_two_qblocks": (2, ("full", (4, 4, 4)), 8, 2, 128, (0, 777), 800, False),
    "r1_d64_three_seqs": (3, ("sparse", (4, 3, 2), 16), 4, 1, 64, (0, 129, 300), 300, False),
    "r2_d64_two_qblocks": (2, ("full", (4, 4, 4)), 8, 2, 64, (100, 257), 260, False),
    "r1_d128_mha": (1, ("sparse", (10, 5, 4, 3, 2), 64), 4, 4, 128, (1024,), 1024, False),
    "r1_d128_root_only": (2, ("sparse", (4, 3), 1), 8, 2, 128, (0, 65), 100, False),
    "r2_d128_341": (1, ("full", (4, 4, 4, 4)), 4, 1, 128, (129,), 200, False),
    "r2_d128_8b_shape": (1, ("sparse", (10, 5, 4, 3), 64), 32, 8, 128, (4096,), 4096, False),
    "r2_d128_fp16_overflow": (2, ("sparse", (10, 5, 4, 3), 64), 32, 8, 128, (700, 64), 768, True),
    "r1_d64_fp16_overflow": (3, ("sparse", (4, 3, 2), 16), 4, 1, 64, (0, 129, 300), 300, True),
    # 512 and more query rows per kv head: eight waves, phase-shifted
    "w8_d128_dense": (1, ("full", (4, 4, 4, 4)), 4, 1, 128, (1000,), 1024, False),
    "w8_d64_two_seqs": (2, ("sparse", (10, 5, 4, 3), 64), 64, 8, 64, (0, 300), 320, False),
    "w8_d128_short_prefix": (1, ("sparse", (10, 5, 4, 3), 64), 16, 2, 128, (20,), 64, False),
    "w8_d128_exact_blocks": (2, ("sparse", (10, 5, 4, 3), 64), 16, 2, 128, (256, 129), 256, False),
    "w8_d128_fp16_overflow": (2, ("sparse", (10, 5, 4, 3), 64), 64, 8, 128, (700, 64), 768, True),
    # the key split shared out over ragged sequences: more sequences than one wave's lanes,
    # a tree larger than the shortest chunk, and a batched grouped-query layout
    "many_seqs_d64": (70, ("sparse", (4, 3, 2), 16), 4, 1, 64, tuple((37 * i) % 301 for i in range(70)), 300,
                      False),
    "w4_d128_tree341_short": (3, ("full", (4, 4, 4, 4)), 2, 2, 128, (0, 40, 700), 704, False),
    "w8_batched_ragged": (8, ("sparse", (10, 5, 4, 3), 64), 16, 2, 128, (1006, 3549, 2810, 496, 1215, 1801, 1667,
                                                                   2011), 3584, False),
}


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from speculative_decoding_amd import lib
    lib()
    return torch.device("cuda:0")


def _plans(tree, seed):
    from speculative_decoding_amd import medusa as M
    if tree[0] == "full":
        return oracle.plan_full(tree[1]), M.medusa_tree_plan_full(tree[1])
    widths, n = tree[1], tree[2]
    rng = np.random.default_rng(seed)
    acc = np.zeros((len(widths), max(widths)))
    for k, w in enumerate(widths):
        acc[k, :w] = np.sort(rng.uniform(0.01, 0.3, size=w))[::-1]
    return (oracle.plan_from_accuracy(acc, widths, n),
            M.medusa_tree_plan_from_accuracy(acc, widths, n))


def _big_values(v, seed, tag):
    """Put values beyond fp16's range (about +-9e4, still exact in bf16) at a few seeded
    places of a bf16 tensor (bit patterns)."""
    from synth import f32_to_bf16_bits
    flat = v.reshape(-1)
    idx = integers(seed, tag + ".big", 0, flat.size, (max(1, flat.size // 5000),))
    sign = np.where(integers(seed, tag + ".sign", 0, 2, idx.shape) > 0, 1.0, -1.0)
    flat[idx] = f32_to_bf16_bits((sign * 9.0e4).astype(np.float32))


@pytest.mark.parametrize("name", sorted(CASES))
def test_tree_attention(dev, name):
    import torch
    from speculative_decoding_amd import medusa as M
    from speculative_decoding_amd.step import host_to_device
    B, tree, Hq, Hkv, d, lens, Lcap, big = CASES[name]
    seed = sorted(CASES).index(name)
    oplan, gplan = _plans(tree, seed)
    N = oplan.n_nodes
    say(f"[attention {name}] B={B} N={N} Hq={Hq} Hkv={Hkv} d={d} lens={lens} Lcap={Lcap}")
    q = normal_bf16(seed, "attn.q", (B, N, Hq, d), 1.0)
    kt = normal_bf16(seed, "attn.kt", (B, N, Hkv, d), 1.0)
    vt = normal_bf16(seed, "attn.vt", (B, N, Hkv, d), 1.0)
    kc = normal_bf16(seed, "attn.kc", (B, Lcap, Hkv, d), 1.0)
    vc = normal_bf16(seed, "attn.vc", (B, Lcap, Hkv, d), 1.0)
    if big:
        _big_values(vc, seed, "attn.vc")
        _big_values(vt, seed, "attn.vt")
    L = np.asarray(lens, dtype=np.int32)
    want = oracle.tree_attention(oplan, oracle.as_f64(q, "bf16"), oracle.as_f64(kt, "bf16"),
                                 oracle.as_f64(vt, "bf16"), kc, vc, L, "bf16")
    gplan.upload(dev)
    D = lambda a: host_to_device(a, "bf16", dev)
    out = torch.empty((B, N, Hq, d), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(M.medusa_attention_workspace(gplan, "bf16", B, Hq, Hkv, d, Lcap),
                     dtype=torch.uint8, device=dev)
    M.medusa_tree_attention(gplan, "bf16", B, Hq, Hkv, d, Lcap, 0.0, D(q), D(kt), D(vt), D(kc),
                            D(vc), torch.as_tensor(L, device=dev), out, ws)
    torch.cuda.synchronize()
    close(f"{name} o", out.float().cpu().numpy(), want)
