"""Pins of the CPU oracle against things other than itself: the page's printed output,
closed forms, brute force on tiny inputs, and library routines on special cases."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import make_inputs
from synth.gen import accuracy_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LN3, LN7 = math.log(3.0), math.log(7.0)
# exact SiLU values: sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4, sigma(ln 7) = 7/8
SILU_CLOSED = {0.0: 0.0, LN3: 0.75 * LN3, -LN3: -0.25 * LN3, LN7: 0.875 * LN7, -LN7: -0.125 * LN7}


def f32(x):
    return np.asarray(x, dtype=np.float32)


# ------------------------------------------------------------------ heads

def test_zero_init_matches_printed_example():
    """Page example: zero-initialised FF layer + projection copied from lm_head makes every
    head reproduce lm_head exactly; the page prints [True, True, True]."""
    g = json.load(open(os.path.join(GOLDEN, "page_zero_init_example.json")))
    inp = make_inputs("tiny", 0, zero_init=True)
    assert (inp.cfg.H, inp.cfg.V, inp.cfg.K) == (g["hidden_size"], g["vocab_size"], g["num_heads"])
    logits, ids, _, _ = oracle.heads_forward(inp.h, inp.w1, inp.b1, inp.w2, inp.cfg.s, "f32")
    lm = oracle.lm_head_logits(inp.w_lm, oracle.as_f64(inp.h, "f32"), "f32")
    printed = [bool(np.array_equal(logits[0, k], lm[0])) for k in range(inp.cfg.K)]
    assert printed == g["printed"]
    for k in range(inp.cfg.K):
        np.testing.assert_array_equal(ids[0, k, : inp.cfg.s[k]], oracle.topk(lm[0], inp.cfg.s[k]))


def test_zero_init_bf16_bitwise():
    inp = make_inputs("small", 1, zero_init=True)
    logits, _, _, u = oracle.heads_forward(inp.h, inp.w1, inp.b1, inp.w2, inp.cfg.s, "bf16")
    lm = oracle.lm_head_logits(inp.w_lm, oracle.as_f64(inp.h, "bf16"), "bf16")
    for k in range(inp.cfg.K):
        assert np.array_equal(logits[0, k], lm[0])
        assert np.array_equal(u[0, k], oracle.as_f64(inp.h, "bf16")[0])


def test_heads_bias_silu_closed_form():
    """W1 = 0, b1 with entries whose SiLU is known exactly, W2 = identity:
    logits = h + SiLU(b1) (fp32 rounding of the stored bias aside)."""
    H = 32
    vals = list(SILU_CLOSED)
    b1 = f32([[vals[i % 5] for i in range(H)]])
    h = f32(np.linspace(-1, 1, H))[None, :]
    w1 = np.zeros((1, H, H), np.float32)
    w2 = np.eye(H, dtype=np.float32)[None]
    logits, ids, _, u = oracle.heads_forward(h, w1, b1, w2, [3], "f32")
    want = h[0].astype(np.float64) + np.array([SILU_CLOSED[vals[i % 5]] for i in range(H)])
    np.testing.assert_allclose(logits[0, 0], want, rtol=1e-6, atol=1e-6)


def test_heads_w1_orientation_and_residual():
    """W1 = permutation matrix P (P[i, p(i)] = 1): z_i = h_{p(i)}, so u_i = h_i + SiLU(h_{p(i)}).
    A transposed W1 would use p^-1; a dropped residual would lose h_i."""
    H = 40
    rng = np.random.default_rng(3)
    keys = list(SILU_CLOSED)
    h = f32([keys[i] for i in rng.integers(0, 5, size=H)])[None, :]
    perm = rng.permutation(H)
    assert not np.array_equal(perm, np.argsort(perm))
    w1 = np.zeros((1, H, H), np.float32)
    w1[0, np.arange(H), perm] = 1.0
    b1 = np.zeros((1, H), np.float32)
    V = 7
    sel = rng.integers(0, H, size=V)
    w2 = np.zeros((1, V, H), np.float32)
    w2[0, np.arange(V), sel] = 1.0                  # logits_v = u[sel_v]
    logits, _, _, u = oracle.heads_forward(h, w1, b1, w2, [2], "f32")
    hd = h[0].astype(np.float64)
    u_want = np.array([hd[i] + SILU_CLOSED[float(h[0, perm[i]])] if float(h[0, perm[i]]) in SILU_CLOSED
                       else np.nan for i in range(H)])
    # h values are float32 roundings of the keys; match them back to their exact key
    u_want = np.array([hd[i] + SILU_CLOSED[min(keys, key=lambda k: abs(k - float(h[0, perm[i]])))]
                       for i in range(H)])
    np.testing.assert_allclose(u[0, 0], u_want, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(logits[0, 0], u_want[sel], rtol=1e-6, atol=1e-6)


def test_silu_closed_forms_and_library():
    import torch
    for x, y in SILU_CLOSED.items():
        assert oracle.silu(np.array([x]))[0] == pytest.approx(y, rel=1e-15, abs=1e-300)
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    big = np.array([50.0, -50.0, 800.0, -800.0])
    got = oracle.silu(big)
    assert got[0] == pytest.approx(50.0, rel=1e-15) and abs(got[1]) < 1e-19
    assert got[2] == 800.0 and got[3] == 0.0
    x = np.random.default_rng(0).normal(0, 4, 1000)
    lib = torch.nn.functional.silu(torch.tensor(x, dtype=torch.float64)).numpy()
    np.testing.assert_allclose(oracle.silu(x), lib, rtol=1e-14, atol=1e-300)


# ------------------------------------------------------------------ selection

def test_topk_against_sorted_with_ties():
    rng = np.random.default_rng(1)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        v = rng.integers(-3, 4, size=n).astype(np.float64)   # many ties
        k = int(rng.integers(1, n + 1))
        want = sorted(range(n), key=lambda i: (-v[i], i))[:k]
        assert list(oracle.topk(v, k)) == want


def test_argmax_lowest_against_loop():
    rng = np.random.default_rng(2)
    for _ in range(200):
        v = rng.integers(-2, 3, size=int(rng.integers(1, 30))).astype(np.float64)
        best = 0
        for i in range(len(v)):
            if v[i] > v[best]:
                best = i
        assert oracle.argmax_lowest(v) == best


# ------------------------------------------------------------------ rounding

def test_round_bf16_matches_torch_on_fp32_values():
    import torch
    x = np.random.default_rng(4).normal(0, 3, 20000).astype(np.float32)
    x = np.concatenate([x, np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0])])
    want = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_act(x.astype(np.float64), "bf16"), want)


def test_round_bf16_brute_force_fp64():
    """Nearest bf16 value with ties to even, found by scanning neighbouring bf16 values."""
    rng = np.random.default_rng(5)
    x = rng.normal(0, 1, 3000) * np.exp2(rng.integers(-20, 20, 3000))
    x = np.concatenate([x, [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2.0 - 2 ** -9]])
    got = oracle.round_act(x, "bf16")
    for xi, gi in zip(x, got):
        b = int(np.float32(xi).view(np.uint32) >> 16)
        cands = []
        for c in range(b - 2, b + 3):
            val = float(np.uint32((c & 0xFFFF) << 16).view(np.float32))
            cands.append((abs(val - xi), c & 1, val))
        best = min(cands)
        assert gi == best[2], (xi, gi, best)
    assert oracle.round_act(np.array([1.0 + 2 ** -8]), "bf16")[0] == 1.0
    assert oracle.round_act(np.array([1.0 + 3 * 2 ** -8]), "bf16")[0] == 1.0 + 2 ** -6


# ------------------------------------------------------------------ tree fill

def test_build_tree_page_example():
    g = json.load(open(os.path.join(GOLDEN, "page_tree_example.json")))
    plan = oracle.plan_full(g["top_k"])
    assert len(plan.leaves()) == g["candidates"]
    topk = np.array([[[11, 12, -1], [21, 22, 23]]])
    tokens, pos = oracle.build_tree(plan, np.array([7]), topk, np.array([5]))
    assert tokens[0].tolist() == [7, 11, 12, 21, 22, 23, 21, 22, 23]
    assert pos[0].tolist() == [5, 6, 6, 7, 7, 7, 7, 7, 7]


# ------------------------------------------------------------------ tree attention

def _brute_branch_attention(plan, q, kt, vt, kc, vc, L, scale):
    """Each node's branch run on its own as a causal sequence [prefix; root..node]: the
    newest token's attention over every row, with an explicit loop."""
    B, N, Hq, d = q.shape
    Hkv = kt.shape[2]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        for i in range(N):
            path = plan.path_nodes(i)
            for j in range(Hq):
                g = j // G
                keys = [kc[b, t, g] for t in range(L[b])] + [kt[b, m, g] for m in path]
                vals = [vc[b, t, g] for t in range(L[b])] + [vt[b, m, g] for m in path]
                s = [float(np.dot(q[b, i, j], kk)) * scale for kk in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = sum(w)
                acc = np.zeros(d)
                for wi, vv in zip(w, vals):
                    acc += wi * vv
                out[b, i, j] = acc / tot
    return out


def _rand_attn(rng, B, N, Hq, Hkv, d, Lcap):
    q = rng.normal(size=(B, N, Hq, d))
    kt = rng.normal(size=(B, N, Hkv, d))
    vt = rng.normal(size=(B, N, Hkv, d))
    kc = rng.normal(size=(B, Lcap, Hkv, d)).astype(np.float32)
    vc = rng.normal(size=(B, Lcap, Hkv, d)).astype(np.float32)
    return q, kt, vt, kc, vc


@pytest.mark.parametrize("tree_s,L", [((2, 3), 0), ((2, 3), 1), ((3, 2, 2), 7), ((1, 1, 1), 32),
                                      ((4,), 5)])
def test_tree_attention_equals_branches(tree_s, L):
    rng = np.random.default_rng(len(tree_s) * 100 + L)
    plan = oracle.plan_full(tree_s)
    B, Hq, Hkv, d = 2, 4, 2, 8
    q, kt, vt, kc, vc = _rand_attn(rng, B, plan.n_nodes, Hq, Hkv, d, max(L, 1))
    lens = np.array([L, max(L - 1, 0)])
    got = oracle.tree_attention(plan, q, kt, vt, kc, vc, lens, "f32")
    want = _brute_branch_attention(plan, q, kt, vt, kc.astype(np.float64), vc.astype(np.float64),
                                   lens, 1 / math.sqrt(d))
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7)


def test_tree_attention_sparse_random_plans():
    rng = np.random.default_rng(9)
    for trial in range(6):
        acc = np.sort(rng.uniform(0.05, 0.9, size=(3, 4)), axis=1)[:, ::-1]
        plan = oracle.plan_from_accuracy(acc, (4, 3, 2), int(rng.integers(2, 17)))
        q, kt, vt, kc, vc = _rand_attn(rng, 1, plan.n_nodes, 2, 1, 4, 9)
        lens = np.array([int(rng.integers(0, 10))])
        got = oracle.tree_attention(plan, q, kt, vt, kc, vc, lens, "f32")
        want = _brute_branch_attention(plan, q, kt, vt, kc.astype(np.float64),
                                       vc.astype(np.float64), lens, 0.5)
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-7)


def test_chain_tree_is_causal_sdpa_with_gqa():
    """All top-k = 1: the tree is one chain, so tree attention is ordinary causal attention
    of the chain's tokens after the prefix (torch SDPA, float64, kv heads repeated)."""
    import torch
    rng = np.random.default_rng(11)
    plan = oracle.plan_full((1, 1, 1, 1))
    N, Hq, Hkv, d, L = plan.n_nodes, 6, 2, 16, 13
    q, kt, vt, kc, vc = _rand_attn(rng, 1, N, Hq, Hkv, d, L)
    got = oracle.tree_attention(plan, q, kt, vt, kc, vc, np.array([L]), "f32")
    K = np.concatenate([kc[0].astype(np.float64), kt[0]], 0)     # [L+N, Hkv, d]
    V = np.concatenate([vc[0].astype(np.float64), vt[0]], 0)
    Qt = torch.tensor(q[0]).transpose(0, 1)[None]                # [1, Hq, N, d]
    Kt = torch.tensor(K).transpose(0, 1).repeat_interleave(Hq // Hkv, 0)[None]
    Vt = torch.tensor(V).transpose(0, 1).repeat_interleave(Hq // Hkv, 0)[None]
    mask = torch.ones(N, L + N, dtype=torch.bool).tril(diagonal=L)
    ref = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, attn_mask=mask)
    want = ref[0].transpose(0, 1).numpy()
    np.testing.assert_allclose(got[0], want, rtol=1e-6, atol=1e-7)


def test_tree_attention_special_cases():
    rng = np.random.default_rng(12)
    plan = oracle.plan_full((2, 2))
    q, kt, vt, kc, vc = _rand_attn(rng, 1, plan.n_nodes, 2, 2, 4, 4)
    # empty prefix: the root sees only itself
    got = oracle.tree_attention(plan, q, kt, vt, kc, vc, np.array([0]), "f32")
    np.testing.assert_allclose(got[0, 0], oracle.round_act(vt[0, 0], "f32"), rtol=0, atol=0)
    # equal keys everywhere: uniform weights, output is the mean of the visible values
    kt[:] = 0.3
    kc[:] = np.float32(0.3)
    got = oracle.tree_attention(plan, q, kt, vt, kc, vc, np.array([4]), "f32")
    for i in range(plan.n_nodes):
        vis = np.concatenate([vc[0].astype(np.float64), vt[0, plan.path_nodes(i)]], 0)
        np.testing.assert_allclose(got[0, i], vis.mean(0), rtol=1e-6, atol=1e-7)


# ------------------------------------------------------------------ verifier layer

def test_proxy_qkv_and_out_selection_matrices():
    rng = np.random.default_rng(13)
    V, H, Hq, Hkv, d = 11, 8, 2, 1, 4
    embed = rng.normal(size=(V, H)).astype(np.float32)
    selq = rng.integers(0, H, size=Hq * d)
    selk = rng.integers(0, H, size=Hkv * d)
    wq = np.zeros((Hq * d, H), np.float32); wq[np.arange(Hq * d), selq] = 1
    wk = np.zeros((Hkv * d, H), np.float32); wk[np.arange(Hkv * d), selk] = 2
    wv = np.zeros((Hkv * d, H), np.float32); wv[np.arange(Hkv * d), selk] = -1
    tokens = np.array([[3, 7, 0]])
    x, q, k, v = oracle.proxy_qkv(tokens, embed, wq, wk, wv, Hq, Hkv, d, "f32")
    e = embed[tokens[0]].astype(np.float64)
    np.testing.assert_array_equal(x[0], e)
    np.testing.assert_array_equal(q[0].reshape(3, -1), e[:, selq])          # head-major rows
    np.testing.assert_array_equal(k[0].reshape(3, -1), 2 * e[:, selk])
    np.testing.assert_array_equal(v[0].reshape(3, -1), -e[:, selk])
    o = rng.normal(size=(1, 3, Hq, d)).astype(np.float32).astype(np.float64)
    selo = rng.integers(0, Hq * d, size=H)
    wo = np.zeros((H, Hq * d), np.float32); wo[np.arange(H), selo] = 1
    nh = oracle.proxy_out(x, o, wo, "f32")
    np.testing.assert_array_equal(nh[0], oracle.round_act(e + o[0].reshape(3, -1)[:, selo], "f32"))


def test_verify_selection_matrix():
    rng = np.random.default_rng(14)
    V, H = 9, 6
    sel = rng.integers(0, H, size=V)
    c = rng.uniform(0.5, 2.0, size=V).astype(np.float32)
    w = np.zeros((V, H), np.float32); w[np.arange(V), sel] = c
    nh = rng.normal(size=(1, 4, H))
    logits, am = oracle.verify(nh, w, "f32")
    want = c.astype(np.float64)[None, :] * nh[0][:, sel]
    np.testing.assert_allclose(logits[0], want, rtol=1e-15)
    assert am[0].tolist() == [int(np.argmax(r)) for r in want]


# ------------------------------------------------------------------ acceptance

def test_accept_hand_cases():
    plan = oracle.plan_full((2, 3))   # nodes: 0; (0,)=1 (1,)=2; (0,x)=3..5; (1,x)=6..8
    tokens = np.array([[5, 10, 11, 20, 21, 22, 20, 21, 22]])
    # root chooses 11 -> node 2; node 2 chooses 21 -> node 7; node 7 chooses 99
    am = np.array([[11, 0, 21, 0, 0, 0, 0, 99, 0]])
    a, nodes, toks = oracle.accept(plan, tokens, am)
    assert a.tolist() == [2] and nodes[0].tolist() == [0, 2, 7] and toks[0].tolist() == [11, 21, 99]
    # nothing accepted: only the root's own choice is emitted
    am = np.array([[42, 20, 21, 0, 0, 0, 0, 0, 0]])
    a, nodes, toks = oracle.accept(plan, tokens, am)
    assert a.tolist() == [0] and nodes[0].tolist() == [0, -1, -1] and toks[0].tolist() == [42, -1, -1]
    # a child would match, but its parent was rejected: depth stays 1
    am = np.array([[10, 77, 20, 0, 0, 0, 0, 0, 0]])
    a, nodes, toks = oracle.accept(plan, tokens, am)
    assert a.tolist() == [1] and nodes[0].tolist() == [0, 1, -1] and toks[0].tolist() == [10, 77, -1]


@pytest.mark.parametrize("cfg,seed", [("tiny", s) for s in range(6)] + [("small_batched", 0),
                                                                         ("small", 1),
                                                                         ("small_rope", 0),
                                                                         ("small_rope", 2)])
def test_step_equals_greedy_decoding(cfg, seed):
    """Emitted tokens equal plain greedy decoding with the same verifier, and the accepted
    length is maximal ("Medusa Decoding Heads", section "Diepe duik")."""
    from tests import planting
    inp = planting.planted_inputs(cfg, seed)
    plan = planting.plan_for(inp.cfg, inp.acc)
    res = oracle.step(inp, plan)
    for b in range(inp.cfg.B):
        a = int(res.accept_len[b])
        g, _, _ = oracle.greedy_decode(inp, b, int(res.root[b]), a + 1)
        assert res.accept_tokens[b, : a + 1].tolist() == g.tolist()
        if a < plan.max_depth:
            node = int(res.accept_nodes[b, a])
            kids = [i for i in range(plan.n_nodes) if plan.parent[i] == node]
            assert int(g[a]) not in {int(res.tokens[b, i]) for i in kids}


@pytest.mark.parametrize("cfg,seed", [("tiny_loop", 0), ("tiny_loop", 2), ("small_loop", 1),
                                      ("small_loop", 3), ("small_rope_loop", 0),
                                      ("small_rope_loop", 1)])
def test_decode_loop_equals_greedy_decoding(cfg, seed):
    """Several rounds, each keeping the longest accepted branch and feeding its last
    hidden state to the heads (glossary "Medusa Heads", section "Attention arborescente
    et acceptation"), emit exactly the plain greedy stream ("Medusa Decoding Heads",
    section "Diepe duik"), and the cache holds the rows greedy decoding would have
    appended."""
    from tests import planting
    inp = planting.planted_inputs(cfg, seed)
    plan = planting.plan_for(inp.cfg, inp.acc)
    root0, streams, res = oracle.decode_loop(inp, plan, 4)
    assert any(int(r.accept_len.max()) > 0 for r in res)      # some branch longer than the root
    for b in range(inp.cfg.B):
        g, _, _ = oracle.greedy_decode(inp, b, int(root0[b]), len(streams[b]))
        assert streams[b].tolist() == g.tolist()
    # the cache after the rounds: prefix unchanged, then the root and each round's accepted
    # tokens, with the k/v the verifier computes for them
    cur, root = inp, None
    for r in res:
        cur_next, root = oracle.advance(cur, plan, r)
        for b in range(inp.cfg.B):
            L, a = int(cur.prefix_lens[b]), int(r.accept_len[b])
            assert int(cur_next.prefix_lens[b]) == L + a + 1
            assert np.array_equal(cur_next.k_cache[b, :L], cur.k_cache[b, :L])   # earlier rows kept
            assert np.array_equal(cur_next.v_cache[b, :L], cur.v_cache[b, :L])
            toks = [int(r.tokens[b, 0])] + [int(t) for t in r.accept_tokens[b, :a]]
            _, _, k_ref, v_ref = oracle.proxy_qkv(np.array([toks]), inp.embed, inp.wq, inp.wk, inp.wv,
                                                  inp.cfg.Hq, inp.cfg.Hkv, inp.cfg.d, inp.dtype,
                                                  positions=np.arange(L, L + a + 1)[None],
                                                  rope_base=inp.cfg.rope_base)
            got_k = oracle.as_f64(cur_next.k_cache[b, L: L + a + 1], inp.dtype)
            got_v = oracle.as_f64(cur_next.v_cache[b, L: L + a + 1], inp.dtype)
            assert np.array_equal(got_k, k_ref[0]) and np.array_equal(got_v, v_ref[0])
        cur = cur_next


def test_advance_rejects_a_full_cache():
    from tests import planting
    inp = planting.planted_inputs("tiny", 0)       # Lcap == L: no room for the root's row
    plan = planting.plan_for(inp.cfg, inp.acc)
    res = oracle.step(inp, plan)
    with pytest.raises(ValueError):
        oracle.advance(inp, plan, res)


# ------------------------------------------------------------------ typical acceptance

NEG = -1e30     # a logit whose probability underflows to exactly 0 at any temperature used


@pytest.mark.parametrize("T", [0.05, 0.7, 1.0, 3.0])
def test_softmax_entropy_against_scipy(T):
    from scipy.special import softmax
    from scipy.stats import entropy
    g = np.random.default_rng(11)
    lg = g.normal(size=(3, 5, 257)) * 2.0
    p, H = oracle.softmax_entropy(lg, T)
    np.testing.assert_allclose(p, softmax(lg / T, axis=-1), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(H, entropy(p, axis=-1), rtol=1e-10, atol=1e-13)


def test_softmax_entropy_closed_forms():
    # uniform over m of V tokens: p = 1/m, H = ln m, at any temperature
    for m, T in ((1, 1.0), (4, 0.3), (7, 2.0)):
        lg = np.full(50, NEG)
        lg[[3, 9, 11, 20, 21, 33, 40][:m]] = 1.25
        p, H = oracle.softmax_entropy(lg, T)
        assert abs(H - math.log(m)) < 1e-12
        assert np.allclose(p[lg > NEG], 1.0 / m, rtol=1e-13, atol=0) and p[lg == NEG].max() == 0.0
    # two tokens a, b: p_a = 1 / (1 + e^{-(a-b)/T}), H = binary entropy
    lg = np.full(10, NEG)
    lg[2], lg[5] = 0.9, -0.4
    p, H = oracle.softmax_entropy(lg, 0.5)
    pa = 1.0 / (1.0 + math.exp(-(0.9 + 0.4) / 0.5))
    assert abs(p[2] - pa) < 1e-15 and abs(p[5] - (1.0 - pa)) < 1e-15
    assert abs(H - (-pa * math.log(pa) - (1 - pa) * math.log(1 - pa))) < 1e-14


def _typical_case():
    """The 2x3 tree of the page's example with hand-set distributions (vocabulary 100).
    Nodes: 0 root; 1 = (0,) token 10, 2 = (1,) token 11; 3..5 = (0, r) tokens 20, 21, 22;
    6..8 = (1, r) tokens 20, 21, 22."""
    plan = oracle.plan_full((2, 3))
    tokens = np.array([[5, 10, 11, 20, 21, 22, 20, 21, 22]])
    lg = np.full((1, 9, 100), NEG)
    lg[0, 0, [10, 11]] = 0.0                    # root: 1/2 each, H = ln 2
    lg[0, 1, [20, 21, 22, 23]] = 1.0            # node 1: 1/4 each, H = ln 4
    lg[0, 2, 20] = math.log(9.0)                # node 2: token 20 at 9/10, token 50 at 1/10
    lg[0, 2, 50] = 0.0
    lg[0, 3, 77] = 0.0                          # node 3: all mass on 77
    for i in range(4, 9):
        lg[0, i, 60 + i] = 0.0
    am = np.array([[int(np.argmax(lg[0, i])) for i in range(9)]])
    return plan, tokens, lg, am


def test_typical_accept_hand_case():
    plan, tokens, lg, am = _typical_case()
    # eps 0.3, delta 0.4: tau_root = min(0.3, 0.4/2) = 0.2 < 1/2 -> nodes 1 and 2 pass;
    # tau_1 = min(0.3, 0.4/4) = 0.1 < 1/4 -> nodes 3, 4, 5 pass; under node 2 only token 20
    # (9/10) passes (node 6).  Deepest: depth 2, lowest index: node 3.
    a, nodes, toks, prob, tau = oracle.typical_accept(plan, tokens, lg, am, 1.0, 0.3, 0.4)
    assert a.tolist() == [2] and nodes[0].tolist() == [0, 1, 3] and toks[0].tolist() == [10, 20, 77]
    np.testing.assert_allclose(prob[0], [1, 0.5, 0.5, 0.25, 0.25, 0.25, 0.9, 0, 0], rtol=1e-14,
                               atol=1e-300)
    h2 = -(0.9 * math.log(0.9) + 0.1 * math.log(0.1))
    np.testing.assert_allclose(tau[0, :3], [0.2, 0.1, min(0.3, 0.4 * math.exp(-h2))], rtol=1e-14)
    # a threshold above 1/2 at the root: nothing passes, the root's argmax (lowest id of the
    # tie: 10) is emitted
    a, nodes, toks, _, tau = oracle.typical_accept(plan, tokens, lg, am, 1.0, 0.6, 1.5)
    assert abs(tau[0, 0] - 0.6) < 1e-15
    assert a.tolist() == [0] and nodes[0].tolist() == [0, -1, -1] and toks[0].tolist() == [10, -1, -1]
    # equality does not pass: tau_1 = min(0.25, 10/4) = 1/4 = p of node 1's children, so
    # the branch continues only under node 2 (token 20 at 9/10 > 1/4: node 6)
    a, nodes, toks, prob, tau = oracle.typical_accept(plan, tokens, lg, am, 1.0, 0.25, 10.0)
    assert tau[0, 1] == 0.25 and prob[0, 3] == 0.25
    assert a.tolist() == [2] and nodes[0].tolist() == [0, 2, 6] and toks[0].tolist() == [11, 20, 66]


@pytest.mark.parametrize("cfg,seed", [("tiny", 0), ("tiny", 3), ("small", 1), ("small_batched", 0)])
def test_typical_at_low_temperature_is_greedy(cfg, seed):
    """As T -> 0 the distribution concentrates on the argmax (planted margins >= 1e-2 give
    p(argmax) = 1 and p(other) = 0 in fp64 at T = 1e-6) and its entropy on 0, so a
    candidate passes exactly when it is the argmax: greedy acceptance."""
    from tests import planting
    inp = planting.planted_inputs(cfg, seed)
    plan = planting.plan_for(inp.cfg, inp.acc)
    res = oracle.step(inp, plan)
    a, nodes, toks, prob, _ = oracle.typical_accept(plan, res.tokens, res.logits, res.node_argmax,
                                                    1e-6, 0.3, 0.09)
    assert np.array_equal(a, res.accept_len)
    assert np.array_equal(nodes, res.accept_nodes) and np.array_equal(toks, res.accept_tokens)
    assert set(np.unique(prob).tolist()) <= {0.0, 1.0}


def test_typical_threshold_extremes():
    from tests import planting
    inp = planting.planted_inputs("small_batched", 0)
    plan = planting.plan_for(inp.cfg, inp.acc)
    res = oracle.step(inp, plan)
    # delta = 0: tau = 0 and every finite logit has p > 0, so every node passes; the kept
    # branch ends at the first deepest node
    a, nodes, toks, prob, tau = oracle.typical_accept(plan, res.tokens, res.logits,
                                                      res.node_argmax, 1.0, 0.5, 0.0)
    first_deep = min(i for i in range(plan.n_nodes) if plan.depth[i] == plan.max_depth)
    assert (prob > 0).all() and (tau == 0).all()
    for b in range(inp.cfg.B):
        assert a[b] == plan.max_depth and nodes[b].tolist() == plan.path_nodes(first_deep)
        assert toks[b, -1] == res.node_argmax[b, first_deep]
    # tau above 1: nothing passes; only the root's argmax is emitted
    a, nodes, toks, _, _ = oracle.typical_accept(plan, res.tokens, res.logits, res.node_argmax,
                                                 1.0, 2.0, 1e9)
    assert (a == 0).all() and (toks[:, 0] == res.node_argmax[:, 0]).all()


def test_typical_higher_threshold_never_accepts_more():
    from tests import planting
    inp = planting.planted_inputs("small", 0)
    plan = planting.plan_for(inp.cfg, inp.acc)
    res = oracle.step(inp, plan)
    prev = None
    for eps in (1e-9, 1e-6, 1e-5, 1e-4, 1e-3, 1e-2, 0.1, 1.0):
        a = oracle.typical_accept(plan, res.tokens, res.logits, res.node_argmax, 1.0, eps, 1.0)[0]
        if prev is not None:
            assert (a <= prev).all()
        prev = a


# ------------------------------------------------------------------ rotary positions

def test_rope_closed_forms():
    base, d, p = 10000.0, 8, 7.0
    x = np.zeros((1, d))
    # position 0 is the identity
    g = np.random.default_rng(3).normal(size=(2, 3, d))
    assert np.array_equal(oracle.rope(g, np.zeros(2), base), g)
    # a unit vector at i < d/2 turns towards i + d/2 by p * base^(-2i/d), and back from there
    for i in range(d // 2):
        th = p * base ** (-2.0 * i / d)
        e = x.copy()
        e[0, i] = 1.0
        y = oracle.rope(e, np.array(p), base)[0]
        want = np.zeros(d)
        want[i], want[i + d // 2] = math.cos(th), math.sin(th)
        np.testing.assert_allclose(y, want, rtol=0, atol=1e-15)
        e = x.copy()
        e[0, i + d // 2] = 1.0
        y = oracle.rope(e, np.array(p), base)[0]
        want = np.zeros(d)
        want[i], want[i + d // 2] = -math.sin(th), math.cos(th)
        np.testing.assert_allclose(y, want, rtol=0, atol=1e-15)
    # d = 2: the plane rotation by the position itself (theta_0 = 1)
    v = np.array([[0.3, -1.7]])
    y = oracle.rope(v, np.array(2.5), base)[0]
    c, s = math.cos(2.5), math.sin(2.5)
    np.testing.assert_allclose(y, [0.3 * c + 1.7 * s, -1.7 * c + 0.3 * s], rtol=1e-15)


def test_rope_depends_on_relative_position_only():
    g = np.random.default_rng(5)
    q = g.normal(size=(4, 64))
    k = g.normal(size=(4, 64))
    for m, n, shift in ((3, 0, 1000), (100, 97, 12345), (0, 4096, 7)):
        a = (oracle.rope(q, np.array(m), 10000.0) * oracle.rope(k, np.array(n), 10000.0)).sum(-1)
        b = (oracle.rope(q, np.array(m + shift), 10000.0) *
             oracle.rope(k, np.array(n + shift), 10000.0)).sum(-1)
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)
        np.testing.assert_allclose(np.linalg.norm(oracle.rope(q, np.array(m), 10000.0), axis=-1),
                                   np.linalg.norm(q, axis=-1), rtol=1e-13)


def test_root_only_decode_loop_is_greedy_decoding():
    """A root-only tree accepts nothing and emits the root's argmax each round: the loop
    reduces to plain greedy decoding."""
    from tests import planting
    inp = planting.planted_inputs("small_loop", 1)
    plan = oracle.plan_from_accuracy(inp.acc, inp.cfg.tree_s, 1)
    root0, streams, res = oracle.decode_loop(inp, plan, 5)
    assert all(int(r.accept_len.max()) == 0 for r in res)
    for b in range(inp.cfg.B):
        g, _, _ = oracle.greedy_decode(inp, b, int(root0[b]), 5)
        assert streams[b].tolist() == g.tolist()


# ------------------------------------------------------------------ tree plan (oracle only)
#
# The glossary page "Medusa Heads", section "Attention arborescente et acceptation":
# candidates are the Cartesian product of the heads' best ranks (2 x 3 -> six
# continuations), arranged as a tree with shared prefixes, and a sparse tree keeps the
# most accurate combinations.  These pins use the oracle alone; no library is loaded.

def _popcount(x: int) -> int:
    return bin(int(x)).count("1")


def _downsets_of(widths):
    """Every prefix-closed set of rank tuples of the Cartesian tree with these
    per-depth widths (the root excluded), enumerated by choosing, for every child of
    a chosen node, whether it and which of its own descendants are kept."""
    def below(prefix):
        d = len(prefix)
        if d == len(widths):
            return [[]]
        per_child = []
        for r in range(widths[d]):
            t = prefix + (r,)
            per_child.append([[]] + [[t] + rest for rest in below(t)])
        return [[x for part in combo for x in part] for combo in itertools.product(*per_child)]
    return below(())


def _expected_accept_by_enumeration(paths, acc, widths):
    """E[accepted candidates] with independent heads: head k is right at rank i with
    probability acc[k][i] and at no kept rank otherwise; the walk accepts depth d when
    the tuple of the first d outcomes is in the tree.  Every joint outcome is listed."""
    present = set(tuple(p) for p in paths)
    outcomes = []
    for k, w in enumerate(widths):
        o = [(i, float(acc[k][i])) for i in range(w)]
        o.append((-1, 1.0 - sum(p for _, p in o)))
        outcomes.append(o)
    e = 0.0
    for joint in itertools.product(*outcomes):
        p = 1.0
        for _, pk in joint:
            p *= pk
        a = 0
        for d in range(1, len(widths) + 1):
            t = tuple(r for r, _ in joint[:d])
            if -1 in t or t not in present:
                break
            a = d
        e += p * a
    return e


@pytest.mark.parametrize("widths,nodes,leaves", [((2, 3), 9, 6), ((3, 4, 4, 4), 256, 192),
                                                 ((4, 4, 4, 4), 341, 256), ((5,), 6, 5),
                                                 ((1, 1, 1, 1, 1), 6, 1), ((2, 1, 3), 11, 6)])
def test_plan_full_node_counts(widths, nodes, leaves):
    """Closed forms: a full Cartesian tree has 1 + sum_d prod_{k<=d} s_k nodes and
    prod_k s_k leaves; the page's 2 x 3 example has six candidate continuations."""
    plan = oracle.plan_full(widths)
    assert plan.n_nodes == nodes
    assert len(plan.leaves()) == leaves
    assert plan.max_depth == len(widths)
    assert plan.mask_words == (nodes + 63) // 64
    per_depth = np.bincount(plan.depth, minlength=len(widths) + 1).tolist()
    assert per_depth == [1] + [int(np.prod(widths[:d])) for d in range(1, len(widths) + 1)]


def test_plan_full_page_example_written_out():
    """The 2 x 3 tree, breadth first, written out by hand: the root, head 1's two
    candidates, then head 2's three candidates under each of them."""
    plan = oracle.plan_full((2, 3))
    assert plan.paths == [(), (0,), (1,), (0, 0), (0, 1), (0, 2), (1, 0), (1, 1), (1, 2)]
    assert plan.parent.tolist() == [-1, 0, 0, 1, 1, 1, 2, 2, 2]
    assert plan.depth.tolist() == [0, 1, 1, 2, 2, 2, 2, 2, 2]
    assert plan.rank.tolist() == [-1, 0, 1, 0, 1, 2, 0, 1, 2]
    # node i sees the root, its parent (for depth 2) and itself
    want = [0b1, 0b11, 0b101, 0b1011, 0b10011, 0b100011, 0b1000101, 0b10000101, 0b100000101]
    assert plan.mask_bits()[:, 0].tolist() == want
    assert plan.leaves() == [3, 4, 5, 6, 7, 8]


@pytest.mark.parametrize("widths", [(2, 3), (3, 4, 4, 4), (4, 4, 4, 4), (3, 2, 2, 2, 2, 2, 2)])
def test_plan_mask_bits_follow_parent_chain(widths):
    """Row i of the mask has exactly the nodes on the parent chain from i up to the
    root: popcount = depth + 1, bit i set, and bit j set only for j <= i.  Trees past 64
    nodes check the split over 64-bit words."""
    plan = oracle.plan_full(widths)
    bits = plan.mask_bits()
    assert bits.shape == (plan.n_nodes, (plan.n_nodes + 63) // 64)
    for i in range(plan.n_nodes):
        chain = set()
        j = i
        while j >= 0:
            chain.add(j)
            j = int(plan.parent[j])
        got = {64 * w + b for w in range(bits.shape[1]) for b in range(64)
               if (int(bits[i, w]) >> b) & 1}
        assert got == chain, i
        assert sum(_popcount(x) for x in bits[i]) == plan.depth[i] + 1
        assert max(got) == i


def test_plan_from_accuracy_ties_written_out():
    """Ties broken by depth (shallower first), then by the rank tuple: with accuracies
    that are powers of two, the scores tie exactly.  Scores: (0)=1/2, (1)=1/4, (0,0)=1/4,
    (0,1)=1/8, (1,0)=1/8, (1,1)=1/16."""
    acc = np.array([[0.5, 0.25], [0.5, 0.25]])
    want = {
        1: [()],
        2: [(), (0,)],
        3: [(), (0,), (1,)],                               # (1) before (0,0): shallower
        4: [(), (0,), (1,), (0, 0)],
        5: [(), (0,), (1,), (0, 0), (0, 1)],               # (0,1) before (1,0): tuple order
        6: [(), (0,), (1,), (0, 0), (0, 1), (1, 0)],
        7: [(), (0,), (1,), (0, 0), (0, 1), (1, 0), (1, 1)],
    }
    for n, paths in want.items():
        assert oracle.plan_from_accuracy(acc, (2, 2), n).paths == paths, n
    with pytest.raises(ValueError):
        oracle.plan_from_accuracy(acc, (2, 2), 8)


def _check_prefix_closed_contiguous(plan):
    present = set(plan.paths)
    for t in plan.paths[1:]:
        assert t[:-1] in present, t
        if t[-1] > 0:
            assert t[:-1] + (t[-1] - 1,) in present, t     # sibling ranks are contiguous
    # breadth-first order: depth ascending, then rank tuple ascending
    assert plan.paths == sorted(plan.paths, key=lambda t: (len(t), t))


@pytest.mark.parametrize("widths,seed", [((3, 2, 2), 4), ((2, 3, 2), 5), ((2, 2, 2, 1), 6)])
def test_plan_from_accuracy_is_best_prefix_closed_tree(widths, seed):
    """Brute force over every prefix-closed node set of a small Cartesian tree: at every
    size, the most-accurate selection has the largest expected accepted length (each set's
    E[a] found by listing every joint outcome of the heads), and it is prefix-closed with
    contiguous sibling ranks."""
    rng = np.random.default_rng(seed)
    acc = np.zeros((len(widths), max(widths)))
    for k, w in enumerate(widths):
        raw = np.sort(rng.uniform(0.02, 0.5, size=w))[::-1]
        acc[k, :w] = raw * (0.9 / raw.sum())                # a miss keeps some mass
    best = {}
    for ds in _downsets_of(widths):
        e = _expected_accept_by_enumeration(ds, acc, widths)
        best[len(ds)] = max(best.get(len(ds), -1.0), e)
    n_cands = len(oracle.candidate_tuples(widths))
    assert sorted(best) == list(range(n_cands + 1))
    for n_paths, e in best.items():
        plan = oracle.plan_from_accuracy(acc, widths, n_paths + 1)
        assert plan.n_nodes == n_paths + 1
        _check_prefix_closed_contiguous(plan)
        got = _expected_accept_by_enumeration(plan.paths[1:], acc, widths)
        assert abs(got - e) < 1e-12, (n_paths, got, e)


def test_plan_from_accuracy_on_the_workload_tables():
    """The benchmark's 64-node sparse trees: prefix-closed, contiguous, at most one node
    per rank tuple, depth bounded by the heads, and the whole Cartesian tree when every
    candidate is asked for."""
    from synth import get_config
    for name in ("mid", "8b", "batched70b"):
        cfg = get_config(name)
        acc = accuracy_table(cfg, 0)
        plan = oracle.plan_from_accuracy(acc, cfg.tree_s, cfg.n_nodes)
        assert plan.n_nodes == cfg.n_nodes
        _check_prefix_closed_contiguous(plan)
        assert plan.max_depth <= len(cfg.tree_s)
        assert all(t[d] < cfg.tree_s[d] for t in plan.paths for d in range(len(t)))
    full = oracle.plan_from_accuracy(accuracy_table(get_config("8b"), 0), (3, 2, 2), 1 + 3 + 6 + 12)
    assert full.paths == oracle.plan_full((3, 2, 2)).paths
