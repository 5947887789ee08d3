"""One Medusa decode step in fp64 numpy (oracle side).

Arithmetic is done in float64 on the exact values of the stored bf16/fp32
input bits.  Activations are rounded back to the workload's dtype (bf16 with
round-to-nearest-even, or fp32) at the points where a real kernel stores them:
the head hidden u_k, the verifier's q/k/v, the attention output o and the node
hidden state.  Logits and top-k values stay unrounded (they are fp32 outputs on
the device, compared with a tolerance).

Steps and the passages they follow:

* ``heads_forward``   — glossary page "Medusa Heads", section "Comment les
  têtes prédisent les tokens suivants": head k reads the same last hidden
  state h as lm_head, applies one feed-forward layer with SiLU and a residual
  connection, then a projection to the vocabulary:
  logits_k = W2_k (h + SiLU(W1_k h + b1_k)).  lm_head scores t+1, head k
  scores t+k+1.
* ``topk``            — section "Attention arborescente et acceptation": the
  best hypotheses of each head (ordered by logit, ties to the lower id).
* ``build_tree``      — same section: node tokens of the Cartesian tree;
  node 0 carries the base model's own next token.
* ``proxy_qkv``, ``proxy_out`` — the one-layer stand-in for the frozen base
  model that scores the tree (embedding gather, Q/K/V projections, attention
  output projection with residual).  Not part of the method; no norm, MLP or
  bias.  Optionally ``rope`` rotates q and k by position (positions L + depth,
  siblings sharing one); the pages say nothing of positions, so this is the
  common rotary form of decoder layers, off unless a base is given.
* ``tree_attention``  — same section: all candidates are appended at once and
  a mask lets each token see only its tree ancestors (read: ancestors and
  itself) on top of the KV prefix.
* ``verify``          — lm_head on every node, greedy argmax (lowest id wins
  ties): section "Attention arborescente et acceptation", greedy decoding
  accepts a candidate when it matches the model's first choice.
* ``accept``          — the longest accepted branch is kept; its deepest node's
  argmax is emitted after it (the blog page "Medusa no contexto de LLMs",
  section "o que significa medusa na prática de deploy": on rejection, fall
  back to the conventionally generated token).
* ``softmax_entropy``, ``typical_accept`` — typical acceptance for sampling
  (glossary, section "Attention arborescente et acceptation": keep every
  candidate whose probability under the base model exceeds a threshold tied
  to the entropy of that distribution).  The page gives no formula; the
  readings are in ``typical_accept``'s docstring.
* ``advance``, ``decode_loop`` — the next round: the longest accepted branch is
  kept and its last hidden state feeds the heads (glossary, section "Attention
  arborescente et acceptation").  The branch's rows join the KV cache, the
  deepest accepted node's hidden state becomes the next h and its argmax (the
  emitted bonus token) the next root.
* ``greedy_decode``   — the definition the step must reproduce: plain
  step-by-step greedy decoding with the same verifier ("Medusa Decoding
  Heads", section "Diepe duik": accepted text is exactly what greedy decoding
  would have produced).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

from .plan_ref import TreePlan

__all__ = [
    "as_f64", "round_act", "silu", "matvec_rows", "heads_forward", "lm_head_logits", "topk",
    "argmax_lowest", "build_tree", "proxy_qkv", "tree_attention", "proxy_out", "verify",
    "accept", "greedy_decode", "StepResult", "step", "causal_attention_last", "store_act",
    "advance", "decode_loop", "softmax_entropy", "typical_accept", "typical_branch", "rope",
]

_CHUNK_ROWS = 8192


# ----------------------------------------------------------------- number formats

def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored tensor bits (bf16 as uint16, or fp32)."""
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 tensors are stored as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), returned as float64.

    bf16 keeps 8 significant bits: for normal numbers this drops the low 45 of
    float64's 52 stored mantissa bits with round-half-to-even; below bf16's
    smallest normal (2^-126) values snap to multiples of 2^-133."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    tiny = np.abs(x) < 2.0 ** -126
    if np.any(tiny):
        q = 2.0 ** -133
        out[tiny] = np.round(x[tiny] / q) * q          # np.round: half to even
    big = ~tiny
    bits = x[big].view(np.uint64)
    drop = np.uint64(45)
    lsb = (bits >> drop) & np.uint64(1)
    bits = (bits + (np.uint64(1) << np.uint64(44)) - np.uint64(1) + lsb) & ~((np.uint64(1) << drop) - np.uint64(1))
    out[big] = bits.view(np.float64)
    return out


def round_act(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the activation dtype (bf16 or fp32) and return float64."""
    if dtype == "bf16":
        return _round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(x) = x / (1 + e^-x), evaluated without overflow for large |x|."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = x[pos] / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = x[~pos] * e / (1.0 + e)
    return out


def matvec_rows(w: np.ndarray, x: np.ndarray, dtype: str) -> np.ndarray:
    """W @ x for a stored [R, C] matrix W and float64 x of shape [C] or [C, M],
    upcasting W to float64 a block of rows at a time."""
    R = w.shape[0]
    out = np.empty((R,) + x.shape[1:], dtype=np.float64)
    for r0 in range(0, R, _CHUNK_ROWS):
        r1 = min(R, r0 + _CHUNK_ROWS)
        out[r0:r1] = as_f64(w[r0:r1], dtype) @ x
    return out


# ----------------------------------------------------------------- selection

def topk(values: np.ndarray, k: int) -> np.ndarray:
    """Ids of the k largest values, ordered by value descending, ties to the lower id."""
    v = np.asarray(values, dtype=np.float64)
    ids = np.arange(v.shape[0])
    order = np.lexsort((ids, -v))   # primary: -v ascending; secondary: id ascending
    return order[:k].astype(np.int64)


def argmax_lowest(values: np.ndarray) -> int:
    """Index of the largest value; the lowest index among equal maxima."""
    return int(np.argmax(np.asarray(values, dtype=np.float64)))


# ----------------------------------------------------------------- heads

def heads_forward(h, w1, b1, w2, s: Sequence[int], dtype: str):
    """Medusa heads on the last hidden state.

    For every sequence b and head k: z = W1_k h_b + b1_k, u = rnd(h_b + SiLU(z)),
    logits = W2_k u; then the top-s_k ids (value descending, lower id on ties).

    Returns (logits [B,K,V], topk_ids [B,K,s_max] (-1 padded),
    topk_vals [B,K,s_max] (0 padded), u [B,K,H])."""
    B, H = h.shape
    K = w1.shape[0]
    V = w2.shape[1]
    s_max = max(s)
    hf = as_f64(h, dtype)
    logits = np.empty((B, K, V))
    ids = np.full((B, K, s_max), -1, dtype=np.int64)
    vals = np.zeros((B, K, s_max))
    u_all = np.empty((B, K, H))
    for k in range(K):
        z = matvec_rows(w1[k], hf.T, dtype).T + as_f64(b1[k], dtype)[None, :]    # [B, H]
        u = round_act(hf + silu(z), dtype)
        u_all[:, k] = u
        logits[:, k] = matvec_rows(w2[k], u.T, dtype).T
        for b in range(B):
            t = topk(logits[b, k], s[k])
            ids[b, k, : s[k]] = t
            vals[b, k, : s[k]] = logits[b, k, t]
    return logits, ids, vals, u_all


def lm_head_logits(w_lm, x: np.ndarray, dtype: str) -> np.ndarray:
    """lm_head applied to float64 rows x [M, H] -> [M, V]."""
    return matvec_rows(w_lm, np.asarray(x, dtype=np.float64).T, dtype).T


# ----------------------------------------------------------------- tree

def build_tree(plan: TreePlan, root_ids: np.ndarray, topk_ids: np.ndarray,
               prefix_lens: np.ndarray):
    """Node tokens: node 0 carries the root token; a depth-d node with rank r
    carries head d's rank-r candidate (head d is 0-based index d-1).  Position
    ids are prefix length + depth (siblings share a position)."""
    B = len(root_ids)
    N = plan.n_nodes
    tokens = np.empty((B, N), dtype=np.int64)
    pos = np.empty((B, N), dtype=np.int64)
    for b in range(B):
        for i in range(N):
            d = int(plan.depth[i])
            tokens[b, i] = root_ids[b] if d == 0 else topk_ids[b, d - 1, plan.rank[i]]
            pos[b, i] = int(prefix_lens[b]) + d
    return tokens, pos


# ----------------------------------------------------------------- verifier layer

def rope(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """Rotary position embedding over the last axis (head dimension d, even), pairing
    element i with element i + d/2: for i < d/2, theta_i = base^(-2i/d) and
    angle = position * theta_i,
        y_i       = x_i cos(angle) - x_{i+d/2} sin(angle)
        y_{i+d/2} = x_{i+d/2} cos(angle) + x_i sin(angle).
    x [..., heads, d]; positions has x's shape without the last two axes."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    theta = np.power(float(base), -2.0 * np.arange(h, dtype=np.float64) / d)
    ang = np.asarray(positions, dtype=np.float64)[..., None, None] * theta     # [..., 1, h]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def proxy_qkv(tokens: np.ndarray, embed, wq, wk, wv, Hq: int, Hkv: int, d: int, dtype: str,
              positions: Optional[np.ndarray] = None, rope_base: float = 0.0):
    """x_i = E[token_i]; q = rnd(Wq x), k = rnd(Wk x), v = rnd(Wv x); with rope_base > 0,
    q and k are then rotated by their positions and rounded again (the projections'
    stored outputs are what the rotation reads).
    tokens [B, N] -> x [B,N,H], q [B,N,Hq,d], k/v [B,N,Hkv,d] (float64)."""
    B, N = tokens.shape
    x = as_f64(embed[tokens.reshape(-1)], dtype)                       # [B*N, H]
    q = round_act(matvec_rows(wq, x.T, dtype).T, dtype).reshape(B, N, Hq, d)
    k = round_act(matvec_rows(wk, x.T, dtype).T, dtype).reshape(B, N, Hkv, d)
    v = round_act(matvec_rows(wv, x.T, dtype).T, dtype).reshape(B, N, Hkv, d)
    if rope_base > 0.0:
        pos = np.asarray(positions).reshape(B, N)
        q = round_act(rope(q, pos, rope_base), dtype)
        k = round_act(rope(k, pos, rope_base), dtype)
    return x.reshape(B, N, -1), q, k, v


def tree_attention(plan: TreePlan, q, k_tree, v_tree, k_cache, v_cache, prefix_lens,
                   dtype: str, scale: Optional[float] = None) -> np.ndarray:
    """Node i, query head j (kv head g = j // (Hq/Hkv), contiguous groups)
    attends to the prefix rows 0..L_b-1 and to the tree rows of its ancestors
    and itself; o = softmax(q k^T * scale) v with scale = 1/sqrt(d), rounded.

    q [B,N,Hq,d]; k_tree/v_tree [B,N,Hkv,d]; k_cache/v_cache [B,Lcap,Hkv,d]
    (stored bits); prefix_lens [B].  Returns o [B,N,Hq,d] float64."""
    B, N, Hq, d = q.shape
    Hkv = k_tree.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((B, N, Hq, d))
    visible = plan.anc[:, None, :]                       # [N, 1, N] broadcast over the group
    for b in range(B):
        L = int(prefix_lens[b])
        kp = as_f64(k_cache[b, :L], dtype)               # [L, Hkv, d]
        vp = as_f64(v_cache[b, :L], dtype)
        for g in range(Hkv):
            qg = q[b, :, g * G:(g + 1) * G, :]           # [N, G, d]
            s_pre = qg @ kp[:, g].T                      # [N, G, L]
            s_tree = qg @ k_tree[b, :, g].T              # [N, G, N]
            s_tree = np.where(visible, s_tree, -np.inf)
            s = np.concatenate([s_pre, s_tree], axis=-1) * scale
            p = np.exp(s - s.max(axis=-1, keepdims=True))
            p /= p.sum(axis=-1, keepdims=True)
            vals = np.concatenate([vp[:, g], v_tree[b, :, g]], axis=0)   # [L+N, d]
            o[b, :, g * G:(g + 1) * G, :] = p @ vals
    return round_act(o, dtype)


def proxy_out(x: np.ndarray, o: np.ndarray, wo, dtype: str) -> np.ndarray:
    """node_hidden = rnd(x + Wo flatten(o)).  x [B,N,H], o [B,N,Hq,d]."""
    B, N, H = x.shape
    of = o.reshape(B * N, -1)
    y = matvec_rows(wo, of.T, dtype).T.reshape(B, N, H)
    return round_act(x + y, dtype)


def verify(node_hidden: np.ndarray, w_lm, dtype: str):
    """lm_head on every tree node and its greedy argmax.
    node_hidden [B,N,H] -> logits [B,N,V], argmax [B,N]."""
    B, N, H = node_hidden.shape
    logits = lm_head_logits(w_lm, node_hidden.reshape(B * N, H), dtype).reshape(B, N, -1)
    am = np.array([[argmax_lowest(logits[b, i]) for i in range(N)] for b in range(B)], dtype=np.int64)
    return logits, am


def accept(plan: TreePlan, tokens: np.ndarray, node_argmax: np.ndarray):
    """Greedy acceptance of the longest branch.

    accepted(root) holds; a node is accepted when its parent is accepted and
    its token equals the parent's argmax.  a = deepest accepted depth, i* the
    accepted node at that depth (unique: siblings carry distinct tokens).
    Emitted tokens: the candidates on the path root -> i* (depths 1..a), then
    i*'s own argmax (the fallback/bonus token).

    Returns accept_len [B], accept_nodes [B, D+1] (root first, -1 padded),
    accept_tokens [B, D+1] (a candidates then the bonus, -1 padded)."""
    B, N = tokens.shape
    D = plan.max_depth
    alen = np.zeros(B, dtype=np.int64)
    anodes = np.full((B, D + 1), -1, dtype=np.int64)
    atoks = np.full((B, D + 1), -1, dtype=np.int64)
    for b in range(B):
        acc = np.zeros(N, dtype=bool)
        acc[0] = True
        for i in range(1, N):     # breadth-first order: parents come first
            p = int(plan.parent[i])
            acc[i] = acc[p] and tokens[b, i] == node_argmax[b, p]
        deepest = max((i for i in range(N) if acc[i]), key=lambda i: (plan.depth[i], -i))
        path = plan.path_nodes(deepest)
        a = len(path) - 1
        alen[b] = a
        anodes[b, : a + 1] = path
        atoks[b, :a] = [tokens[b, i] for i in path[1:]]
        atoks[b, a] = node_argmax[b, deepest]
    return alen, anodes, atoks


# ----------------------------------------------------------------- the definition

def causal_attention_last(q_last: np.ndarray, keys: np.ndarray, vals: np.ndarray,
                          Hq: int, Hkv: int, scale: float) -> np.ndarray:
    """Attention of the newest token over a whole cache (keys/vals [T, Hkv, d]),
    which under a causal mask sees every earlier row and itself.  q_last [Hq, d]."""
    G = Hq // Hkv
    out = np.empty_like(q_last)
    for j in range(Hq):
        g = j // G
        s = keys[:, g] @ q_last[j] * scale
        w = np.exp(s - s.max())
        out[j] = (w[:, None] * vals[:, g]).sum(0) / w.sum()
    return out


def greedy_decode(inp, b: int, first_token: int, n_tokens: int):
    """Plain greedy decoding with the one-layer verifier, one token at a time.

    The cache starts as the prefix of sequence b.  For each step: x = E[tok],
    q/k/v projected and rounded (and q, k rotated to the token's position L + j
    when the workload has a rotary base), (k, v) appended to the cache,
    attention over the whole cache, hidden = rnd(x + Wo o),
    next = argmax(lm_head(hidden)).
    Returns (tokens [n_tokens], hiddens [n_tokens, H], logits [n_tokens, V])
    generated after ``first_token``."""
    cfg = inp.cfg
    dt = inp.dtype
    L = int(inp.prefix_lens[b])
    keys = as_f64(inp.k_cache[b, :L], dt)
    vals = as_f64(inp.v_cache[b, :L], dt)
    scale = 1.0 / np.sqrt(cfg.d)
    tok = int(first_token)
    out_t, out_h, out_l = [], [], []
    base = float(getattr(cfg, "rope_base", 0.0))
    for j in range(n_tokens):
        x = as_f64(inp.embed[tok], dt)
        q = round_act(matvec_rows(inp.wq, x, dt), dt).reshape(cfg.Hq, cfg.d)
        k = round_act(matvec_rows(inp.wk, x, dt), dt).reshape(1, cfg.Hkv, cfg.d)
        v = round_act(matvec_rows(inp.wv, x, dt), dt).reshape(1, cfg.Hkv, cfg.d)
        if base > 0.0:
            q = round_act(rope(q, np.array(L + j), base), dt)
            k = round_act(rope(k, np.array([L + j]), base), dt)
        keys = np.concatenate([keys, k], axis=0)
        vals = np.concatenate([vals, v], axis=0)
        o = round_act(causal_attention_last(q, keys, vals, cfg.Hq, cfg.Hkv, scale), dt)
        hid = round_act(x + matvec_rows(inp.wo, o.reshape(-1), dt), dt)
        lg = matvec_rows(inp.w_lm, hid, dt)
        tok = argmax_lowest(lg)
        out_t.append(tok)
        out_h.append(hid)
        out_l.append(lg)
    return np.array(out_t, dtype=np.int64), np.array(out_h), np.array(out_l)


# ----------------------------------------------------------------- whole step

@dataclass
class StepResult:
    root: np.ndarray            # [B]
    root_logits: np.ndarray     # [B, V]
    head_logits: np.ndarray     # [B, K, V]
    topk_ids: np.ndarray        # [B, K, s_max]
    topk_vals: np.ndarray       # [B, K, s_max]
    u: np.ndarray               # [B, K, H]
    tokens: np.ndarray          # [B, N]
    pos: np.ndarray             # [B, N]
    x: np.ndarray               # [B, N, H]
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    o: np.ndarray               # [B, N, Hq, d]
    node_hidden: np.ndarray     # [B, N, H]
    logits: np.ndarray          # [B, N, V]
    node_argmax: np.ndarray     # [B, N]
    accept_len: np.ndarray
    accept_nodes: np.ndarray
    accept_tokens: np.ndarray

    def as_dict(self) -> Dict[str, np.ndarray]:
        return dict(self.__dict__)


def step(inp, plan: TreePlan, root: Optional[np.ndarray] = None) -> StepResult:
    """One whole decode step on generator inputs ``inp``.  Without ``root`` the
    root token is bootstrapped as argmax(lm_head(h))."""
    cfg = inp.cfg
    dt = inp.dtype
    hf = as_f64(inp.h, dt)
    root_logits = lm_head_logits(inp.w_lm, hf, dt)
    if root is None:
        root = np.array([argmax_lowest(root_logits[b]) for b in range(cfg.B)], dtype=np.int64)
    hl, ids, vals, u = heads_forward(inp.h, inp.w1, inp.b1, inp.w2, cfg.s, dt)
    tokens, pos = build_tree(plan, root, ids, inp.prefix_lens)
    x, q, k, v = proxy_qkv(tokens, inp.embed, inp.wq, inp.wk, inp.wv, cfg.Hq, cfg.Hkv, cfg.d, dt,
                           positions=pos, rope_base=float(getattr(cfg, "rope_base", 0.0)))
    o = tree_attention(plan, q, k, v, inp.k_cache, inp.v_cache, inp.prefix_lens, dt)
    nh = proxy_out(x, o, inp.wo, dt)
    logits, am = verify(nh, inp.w_lm, dt)
    alen, anodes, atoks = accept(plan, tokens, am)
    return StepResult(root=np.asarray(root), root_logits=root_logits, head_logits=hl, topk_ids=ids,
                      topk_vals=vals, u=u, tokens=tokens, pos=pos, x=x, q=q, k=k, v=v, o=o,
                      node_hidden=nh, logits=logits, node_argmax=am, accept_len=alen,
                      accept_nodes=anodes, accept_tokens=atoks)


# ----------------------------------------------------------------- typical acceptance

def softmax_entropy(logits: np.ndarray, temperature: float):
    """The base model's distribution over the vocabulary at temperature T,
    p = softmax(logits / T) along the last axis, and its entropy in nats,
    H = -sum_j p_j ln p_j (0 ln 0 = 0).  Returns (p, H)."""
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    p = e / e.sum(axis=-1, keepdims=True)
    safe = np.where(p > 0.0, p, 1.0)
    H = -(p * np.log(safe)).sum(axis=-1)
    return p, H


def typical_accept(plan: TreePlan, tokens: np.ndarray, logits: np.ndarray,
                   node_argmax: np.ndarray, temperature: float, epsilon: float, delta: float):
    """Typical acceptance of the tree's candidates (glossary, section "Attention
    arborescente et acceptation": for sampling, every candidate whose base-model
    probability exceeds an entropy-linked threshold is kept; more tokens pass
    than under greedy matching, and exact agreement with the base model's
    distribution is given up).

    Readings, since the page gives no formula:
    * node i's base-model distribution is p_i = softmax(logits_i / T) over the
      vocabulary, H_i its entropy in nats (``softmax_entropy``);
    * the threshold falls as the distribution flattens, capped:
      tau_i = min(epsilon, delta * exp(-H_i));
    * a child c of node i is accepted when i is accepted and
      p_i(token_c) > tau_i (strict); several siblings may pass;
    * the kept branch ends at the deepest accepted node, the lowest index among
      equals (breadth-first order puts higher-ranked candidates first); it
      emits its candidates, then that node's most probable token (its argmax),
      as greedy acceptance does.

    Returns accept_len [B], accept_nodes and accept_tokens [B, D+1] (as
    ``accept``), node_prob [B, N] (p of each node's token under its parent's
    distribution; 1 for the root) and node_tau [B, N] (tau_i)."""
    B, N = tokens.shape
    p, H = softmax_entropy(logits, temperature)
    tau = np.minimum(float(epsilon), float(delta) * np.exp(-H))
    prob = np.ones((B, N), dtype=np.float64)
    for b in range(B):
        for i in range(1, N):
            prob[b, i] = p[b, int(plan.parent[i]), int(tokens[b, i])]
    alen, anodes, atoks = typical_branch(plan, tokens, node_argmax, prob, tau)
    return alen, anodes, atoks, prob, tau


def typical_branch(plan: TreePlan, tokens: np.ndarray, node_argmax: np.ndarray,
                   prob: np.ndarray, tau: np.ndarray):
    """The walk of ``typical_accept`` given each node's probability under its parent's
    distribution (prob [B, N]) and each node's threshold (tau [B, N]): node i >= 1 is
    accepted when its parent is and prob[i] > tau[parent]; the kept branch ends at the
    deepest accepted node, the lowest index among equals."""
    B, N = tokens.shape
    D = plan.max_depth
    alen = np.zeros(B, dtype=np.int64)
    anodes = np.full((B, D + 1), -1, dtype=np.int64)
    atoks = np.full((B, D + 1), -1, dtype=np.int64)
    for b in range(B):
        acc = np.zeros(N, dtype=bool)
        acc[0] = True
        for i in range(1, N):     # breadth-first order: parents come first
            par = int(plan.parent[i])
            acc[i] = acc[par] and prob[b, i] > tau[b, par]
        deepest = max((i for i in range(N) if acc[i]), key=lambda i: (plan.depth[i], -i))
        path = plan.path_nodes(deepest)
        a = len(path) - 1
        alen[b] = a
        anodes[b, : a + 1] = path
        atoks[b, :a] = [tokens[b, i] for i in path[1:]]
        atoks[b, a] = node_argmax[b, deepest]
    return alen, anodes, atoks


# ----------------------------------------------------------------- the next round

def store_act(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage form of activation values that are already rounded to ``dtype``: bf16 bit
    patterns (uint16) or float32.  Exact: every input value is representable."""
    if dtype == "bf16":
        f = np.asarray(x, dtype=np.float64).astype(np.float32)
        if not np.array_equal(f.astype(np.float64), np.asarray(x, dtype=np.float64)):
            raise ValueError("value not representable in fp32")
        bits = f.view(np.uint32)
        if np.any(bits & np.uint32(0xFFFF)):
            raise ValueError("value not representable in bf16")
        return (bits >> np.uint32(16)).astype(np.uint16)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def advance(inp, plan: TreePlan, res: StepResult):
    """Commit one step's accepted branch and set up the next round.

    For sequence b with a = accept_len[b] and path = accept_nodes[b, :a+1] (root
    first): the tree K/V rows of the path become KV-cache rows L_b .. L_b + a (they
    are the keys and values greedy decoding computes for those tokens), L_b grows by
    a + 1, the next last hidden state is node_hidden at the path's deepest node, and
    the next root is the emitted bonus token accept_tokens[b, a].

    Returns (inputs for the next step, next roots [B]).  ``inp`` is not modified.
    Raises ValueError when a branch does not fit in the cache (L_b + a + 1 > Lcap)."""
    import copy
    cfg = inp.cfg
    dt = inp.dtype
    nxt = copy.copy(inp)
    nxt.k_cache = inp.k_cache.copy()
    nxt.v_cache = inp.v_cache.copy()
    nxt.prefix_lens = inp.prefix_lens.copy()
    nxt.h = inp.h.copy()
    roots = np.empty(cfg.B, dtype=np.int64)
    for b in range(cfg.B):
        L = int(inp.prefix_lens[b])
        a = int(res.accept_len[b])
        path = [int(i) for i in res.accept_nodes[b, : a + 1]]
        if L + a + 1 > cfg.Lcap:
            raise ValueError(f"sequence {b}: {a + 1} rows do not fit after {L} of {cfg.Lcap}")
        nxt.k_cache[b, L: L + a + 1] = store_act(res.k[b, path], dt)
        nxt.v_cache[b, L: L + a + 1] = store_act(res.v[b, path], dt)
        nxt.prefix_lens[b] = L + a + 1
        nxt.h[b] = store_act(res.node_hidden[b, path[a]], dt)
        roots[b] = int(res.accept_tokens[b, a])
    return nxt, roots


def decode_loop(inp, plan: TreePlan, steps: int):
    """``steps`` whole Medusa steps, each followed by ``advance``; the first bootstraps
    its root as argmax(lm_head(h)).

    Returns (first roots [B], emitted streams: one int64 array per sequence holding
    every step's accepted candidates and bonus token, per-step StepResults)."""
    cur = inp
    root = None
    results = []
    streams = [[] for _ in range(inp.cfg.B)]
    for _ in range(steps):
        res = step(cur, plan, root)
        results.append(res)
        for b in range(inp.cfg.B):
            a = int(res.accept_len[b])
            streams[b].extend(int(t) for t in res.accept_tokens[b, : a + 1])
        cur, root = advance(cur, plan, res)
    return (np.asarray(results[0].root, dtype=np.int64),
            [np.array(t, dtype=np.int64) for t in streams], results)

