"""The C-ABI library on the CPU: it loads, exports every declared symbol, builds the
same tree plans as the oracle, and rejects bad arguments before touching a device."""
import ctypes

import numpy as np
import pytest

import oracle
from synth import CONFIGS, make_inputs
from synth.gen import accuracy_table

M = pytest.importorskip("speculative_decoding_amd.medusa")
from speculative_decoding_amd import header_functions, lib  # noqa: E402


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def test_exports_every_header_symbol():
    L = lib()
    names = header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), f"libmedusa.so does not export {n}"


def _same_plan(cplan, oplan):
    parent, depth, rank, mask = cplan.arrays()
    np.testing.assert_array_equal(parent, oplan.parent)
    np.testing.assert_array_equal(depth, oplan.depth)
    np.testing.assert_array_equal(rank, oplan.rank)
    np.testing.assert_array_equal(mask, oplan.mask_bits())
    assert cplan.info() == (oplan.n_nodes, oplan.max_depth, oplan.mask_words)


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_plan_matches_oracle(name):
    cfg = CONFIGS[name]
    if cfg.tree == "full":
        _same_plan(M.medusa_tree_plan_full(cfg.tree_s), oracle.plan_full(cfg.tree_s))
    else:
        for seed in range(3):
            acc = accuracy_table(cfg, seed)
            _same_plan(M.medusa_tree_plan_from_accuracy(acc, cfg.tree_s, cfg.n_nodes),
                       oracle.plan_from_accuracy(acc, cfg.tree_s, cfg.n_nodes))


def test_plan_from_paths_matches_oracle():
    paths = [(1,), (0,), (0, 2), (0, 0), (1, 0), (0, 0, 3)]
    _same_plan(M.medusa_tree_plan_create(paths), oracle.plan_from_paths(paths))
    _same_plan(M.medusa_tree_plan_create([]), oracle.plan_from_paths([]))


@pytest.mark.parametrize("paths", [[(0, 1)],             # parent (0,) missing
                                   [(0,), (0,)],         # duplicate
                                   [(0,), (64,)]])       # rank beyond the top-k limit
def test_plan_rejects_malformed(paths):
    with pytest.raises(M.MedusaError) as e:
        M.medusa_tree_plan_create(paths)
    assert e.value.status == 4


def test_plan_rejects_rank_after_padding():
    flat = np.array([[0, -1, 2]], np.int32)
    out = ctypes.c_void_p()
    st = lib().medusa_tree_plan_create(flat.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 1, 3,
                                       ctypes.byref(out))
    assert st == 4


def test_plan_too_many_nodes():
    with pytest.raises(M.MedusaError) as e:
        M.medusa_tree_plan_full((64, 64))
    assert e.value.status == 2


# ------------------------------------------------------------------ error paths
FAKE = 1 << 20      # aligned, never dereferenced: every call below fails before any launch


def _heads(**over):
    a = dict(dt=1, B=1, H=256, V=1000, K=3, hidden=FAKE, w1=FAKE, b1=FAKE, w2=FAKE, w_lm=None,
             s=[2, 3, 3], s_max=3, topk_ids=FAKE, topk_vals=FAKE, root=None, u=None, logits=None,
             ws=FAKE, ws_bytes=1 << 40)
    a.update(over)
    s = (ctypes.c_int32 * len(a["s"]))(*a["s"])
    return lib().medusa_heads_forward(a["dt"], a["B"], a["H"], a["V"], a["K"], a["hidden"], a["w1"],
                                      a["b1"], a["w2"], a["w_lm"], s, a["s_max"], a["topk_ids"],
                                      a["topk_vals"], a["root"], a["u"], a["logits"], a["ws"],
                                      a["ws_bytes"], None)


def test_heads_error_paths():
    assert _heads(hidden=None) == 1
    assert _heads(w_lm=FAKE, root=None) == 1
    assert _heads(dt=7) == 3
    assert _heads(H=100) == 2
    assert _heads(K=9) == 2
    assert _heads(s=[2, 65, 3], s_max=65) == 3
    assert _heads(s=[2, 3, 3], s_max=2) == 2
    assert _heads(hidden=FAKE + 8) == 2                    # misaligned
    assert _heads(ws=None) == 5
    assert _heads(ws_bytes=16) == 5
    # at most 2048 vocabulary tiles of 128 rows per head, on every kernel path
    for dt in (0, 1):
        for B in (1, 2, 3, 8, 64):
            assert _heads(dt=dt, B=B, V=262145) == 2, (dt, B)
            assert _heads(dt=dt, B=B, V=262144, ws=None) == 5, (dt, B)


@pytest.mark.skipif(_gpu_visible(), reason="checks the no-device status; a GPU is visible")
def test_no_device_status():
    assert _heads() == 6


def test_workspace_queries_positive():
    assert M.medusa_heads_workspace("bf16", 1, 4096, 128256, 4, 10) > 0
    plan = M.medusa_tree_plan_full((2, 3))
    assert M.medusa_attention_workspace(plan, "bf16", 1, 32, 8, 128, 4096) > 0
    assert M.medusa_verify_workspace(plan, "bf16", 1, 4096, 128256) > 0
    assert M.medusa_attention_workspace(plan, "bf16", 1, 32, 8, 96, 4096) == 0   # d unsupported


def test_tree_and_attention_error_paths():
    plan = M.medusa_tree_plan_full((2, 3))
    s = (ctypes.c_int32 * 3)(2, 3, 3)
    L = lib()
    # not uploaded
    assert L.medusa_build_tree(plan.handle, 1, 3, 3, s, FAKE, FAKE, None, FAKE, None, None) == 8
    # plan deeper than the heads
    assert L.medusa_build_tree(plan.handle, 1, 1, 3, s, FAKE, FAKE, None, FAKE, None, None) == 4
    # plan rank 2 at depth 1 is not < s[0] = 2
    big = M.medusa_tree_plan_full((3, 3))
    assert L.medusa_build_tree(big.handle, 1, 3, 3, s, FAKE, FAKE, None, FAKE, None, None) == 4
    assert L.medusa_tree_attention(plan.handle, 1, 1, 32, 8, 96, 64, 0.0, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == 3
    assert L.medusa_tree_attention(plan.handle, 1, 1, 30, 8, 128, 64, 0.0, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == 2
    assert L.medusa_tree_attention(plan.handle, 1, 1, 32, 8, 128, 64, 0.0, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, FAKE, FAKE, 8, None) == 5
    assert L.medusa_tree_attention(plan.handle, 1, 1, 32, 8, 128, 64, 0.0, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == 8
    assert L.medusa_verify_accept(plan.handle, 1, 1, 4096, 1000, FAKE, FAKE, FAKE, None, FAKE,
                                  None, FAKE, None, FAKE, 1 << 40, None) == 1
    assert L.medusa_verify_accept(plan.handle, 1, 1, 4095, 1000, FAKE, FAKE, FAKE, None, FAKE,
                                  FAKE, FAKE, None, FAKE, 1 << 40, None) == 2
    assert L.medusa_proxy_qkv(1, 9, 256, 1000, 4, 4, 64, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, FAKE, 1 << 40, None) == 1
    assert L.medusa_proxy_out(1, 9, 250, 1000, 4, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40,
                              None) == 2
    assert L.medusa_proxy_qkv(1, 64, 4096, 1000, 32, 8, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              FAKE, FAKE, FAKE, 64, None) == 5
    assert M.medusa_proxy_workspace("bf16", 64, 4096, 32, 8, 128) > 1 << 20
    assert L.medusa_status_string(5) == b"workspace too small"


def _advance(L, plan, **over):
    a = dict(dt=1, B=1, H=256, Hkv=4, d=64, Lcap=64, alen=FAKE, anodes=FAKE, atoks=FAKE,
             kt=FAKE, vt=FAKE, nh=FAKE, kc=FAKE, vc=FAKE, lens=FAKE, hout=FAKE + (1 << 24),
             root=FAKE, over=None)
    a.update(over)
    return L.medusa_advance(plan.handle, a["dt"], a["B"], a["H"], a["Hkv"], a["d"], a["Lcap"],
                            a["alen"], a["anodes"], a["atoks"], a["kt"], a["vt"], a["nh"], a["kc"],
                            a["vc"], a["lens"], a["hout"], a["root"], a["over"], None)


def test_advance_error_paths():
    L = lib()
    plan = M.medusa_tree_plan_full((2, 3))
    assert _advance(L, plan, alen=None) == 1
    assert _advance(L, plan, hout=None) == 1
    assert _advance(L, plan, dt=7) == 3
    assert _advance(L, plan, d=3) == 2                   # K/V row not a multiple of 16 bytes
    assert _advance(L, plan, kc=FAKE + 8) == 2           # misaligned
    assert _advance(L, plan, hout=FAKE) == 2             # next h overlaps node_hidden
    assert _advance(L, plan, Lcap=0) == 2


def test_typical_error_paths():
    from speculative_decoding_amd import medusa as M
    plan = M.medusa_tree_plan_full((2, 3))
    L = lib()
    ws = M.medusa_verify_typical_workspace(plan, "bf16", 2, 256, 1000)
    assert ws > M.medusa_verify_workspace(plan, "bf16", 2, 256, 1000) > 0
    null = None
    # null outputs
    st = L.medusa_verify_accept_typical(plan.handle, 1, 1, 256, 1000, 16, 16, 16, 1.0, 0.1, 0.1,
                                        null, null, null, null, 16, 16, null, 16, ws, null)
    assert st == 1
    # temperature, epsilon, delta out of range (checked before any device access)
    for T, e, d in ((0.0, 0.1, 0.1), (1e-7, 0.1, 0.1), (float("nan"), 0.1, 0.1),
                    (1.0, -0.1, 0.1), (1.0, 0.1, float("inf")), (1.0, float("nan"), 0.1)):
        st = L.medusa_verify_accept_typical(plan.handle, 1, 1, 256, 1000, 16, 16, 16, T, e, d,
                                            null, null, null, 16, 16, 16, null, 16, ws, null)
        assert st == 2, (T, e, d, st)


def test_rope_error_paths():
    L = lib()
    # null pointers, then shapes and bases (all checked before any device access)
    assert L.medusa_rope(1, 4, 2, 1, 64, None, 10000.0, 16, 16, None) == 1
    assert L.medusa_rope(1, 4, 2, 1, 64, 16, 10000.0, None, 16, None) == 1
    for M, Hq, Hkv, d, base in ((0, 2, 1, 64, 1e4), (4, 2, 1, 60, 1e4), (4, 2, 1, 4, 1e4),
                                (4, 0, 1, 64, 1e4), (4, 2, 1, 64, 1.0), (4, 2, 1, 64, float("inf")),
                                (4, 2, 1, 64, float("nan")), (4, 2, 1, 64, -5.0)):
        assert L.medusa_rope(1, M, Hq, Hkv, d, 16, base, 16, 16, None) == 2, (M, Hq, Hkv, d, base)
    # misaligned q for bf16 (8-byte quads)
    assert L.medusa_rope(1, 4, 2, 1, 64, 16, 1e4, 20, 16, None) == 2


def test_probe_error_paths():
    L = lib()
    from speculative_decoding_amd import medusa as M
    assert M.medusa_hbm_probe_bytes(8192 * 3 + 100) == 8192 * 3
    assert M.medusa_hbm_probe_bytes(8191) == 0
    assert L.medusa_hbm_read_probe(None, 1 << 20, 16, None) == 1
    assert L.medusa_hbm_read_probe(16, 1 << 20, None, None) == 1
    assert L.medusa_hbm_read_probe(16, 4096, 16, None) == 2          # under one block
    assert L.medusa_hbm_read_probe(24, 1 << 20, 16, None) == 2       # misaligned
