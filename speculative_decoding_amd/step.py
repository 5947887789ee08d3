"""One Medusa decode step driven through the C ABI.

``MedusaStep`` owns the device buffers of one workload (outputs, intermediates and the
three workspaces, all allocated once through PyTorch) and enqueues the step's calls on
the current stream: heads -> tree -> verifier Q/K/V -> tree attention -> verifier
output -> verify + accept.  It performs no arithmetic of its own.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import numpy as np

from . import medusa as M


def _torch():
    import torch
    return torch


def host_to_device(arr: np.ndarray, dtype: str, device):
    """Upload a generator array: bf16 bit patterns (uint16) or fp32/int32 values."""
    torch = _torch()
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device, non_blocking=False)


def device_weights(inp, device) -> Dict[str, "object"]:
    """Every tensor of a generator draw on the device (plus prefix lengths as int32)."""
    out = {name: host_to_device(arr, inp.dtype, device) for name, arr in inp.tensors().items()}
    out["prefix_lens"] = host_to_device(inp.prefix_lens.astype(np.int32), inp.dtype, device)
    return out


@dataclass
class Dims:
    B: int
    H: int
    V: int
    K: int
    s: Sequence[int]
    Hq: int
    Hkv: int
    d: int
    Lcap: int
    dtype: str
    rope_base: float = 0.0      # rotary positions on the verifier's q and k (0: none)

    @property
    def s_max(self) -> int:
        return max(self.s)

    @classmethod
    def from_config(cls, cfg) -> "Dims":
        return cls(B=cfg.B, H=cfg.H, V=cfg.V, K=cfg.K, s=tuple(cfg.s), Hq=cfg.Hq, Hkv=cfg.Hkv,
                   d=cfg.d, Lcap=cfg.Lcap, dtype=cfg.dtype,
                   rope_base=float(getattr(cfg, "rope_base", 0.0)))


class MedusaStep:
    """``typical``: None for greedy acceptance, or (temperature, epsilon, delta) for typical
    acceptance (medusa_verify_accept_typical)."""

    def __init__(self, dims: Dims, w: Dict[str, "object"], plan: M.TreePlan, device="cuda",
                 keep_logits: bool = False, typical: Optional[Sequence[float]] = None):
        torch = _torch()
        self.dims, self.w, self.plan = dims, w, plan
        self.typical = None if typical is None else tuple(float(x) for x in typical)
        n, D, _ = plan.info()
        self.N, self.D = n, D
        dt = torch.bfloat16 if dims.dtype == "bf16" else torch.float32
        B, H, V, K, s_max = dims.B, dims.H, dims.V, dims.K, dims.s_max
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        act = dict(dtype=dt, device=device)
        self.topk_ids = torch.empty(B, K, s_max, **i32)
        self.topk_vals = torch.empty(B, K, s_max, **f32)
        self.root_ids = torch.zeros(B, **i32)
        self.u = torch.empty(B, K, H, **act)
        self.node_tokens = torch.empty(B, n, **i32)
        self.position_ids = torch.empty(B, n, **i32)
        self.q = torch.empty(B, n, dims.Hq, dims.d, **act)
        self.k_tree = torch.empty(B, n, dims.Hkv, dims.d, **act)
        self.v_tree = torch.empty(B, n, dims.Hkv, dims.d, **act)
        self.o = torch.empty(B, n, dims.Hq, dims.d, **act)
        self.node_hidden = torch.empty(B, n, H, **act)
        self.node_argmax = torch.empty(B, n, **i32)
        self.accept_len = torch.empty(B, **i32)
        self.accept_nodes = torch.empty(B, D + 1, **i32)
        self.accept_tokens = torch.empty(B, D + 1, **i32)
        self.head_logits = torch.empty(B, K + 1, V, **f32) if keep_logits else None
        self.verify_logits = torch.empty(B, n, V, **f32) if keep_logits else None
        u8 = dict(dtype=torch.uint8, device=device)
        self.ws_heads = torch.empty(M.medusa_heads_workspace(dims.dtype, B, H, V, K, s_max), **u8)
        self.ws_attn = torch.empty(M.medusa_attention_workspace(plan, dims.dtype, B, dims.Hq,
                                                                dims.Hkv, dims.d, dims.Lcap), **u8)
        if self.typical is None:
            self.node_prob = self.node_tau = None
            self.ws_verify = torch.empty(M.medusa_verify_workspace(plan, dims.dtype, B, H, V), **u8)
        else:
            self.node_prob = torch.empty(B, n, **f32)
            self.node_tau = torch.empty(B, n, **f32)
            self.ws_verify = torch.empty(M.medusa_verify_typical_workspace(plan, dims.dtype, B, H, V),
                                         **u8)
        self.ws_proxy = torch.empty(M.medusa_proxy_workspace(dims.dtype, B * n, H, dims.Hq,
                                                             dims.Hkv, dims.d), **u8)

    # ---- the four calls plus the verifier layer, in step order
    def heads(self, bootstrap_root: bool = False, keep_u: bool = True):
        d, w = self.dims, self.w
        self.u_written = keep_u
        M.medusa_heads_forward(d.dtype, d.B, d.H, d.V, d.K, w["h"], w["w1"], w["b1"], w["w2"],
                               w["w_lm"] if bootstrap_root else None, d.s, d.s_max, self.topk_ids,
                               self.topk_vals, self.root_ids if bootstrap_root else None,
                               self.u if keep_u else None, self.head_logits, self.ws_heads)

    def tree(self):
        d, w = self.dims, self.w
        M.medusa_build_tree(self.plan, d.B, d.K, d.s_max, d.s, self.root_ids, self.topk_ids,
                            w["prefix_lens"], self.node_tokens, self.position_ids)

    def verifier_in(self):
        d, w = self.dims, self.w
        M.medusa_proxy_qkv(d.dtype, d.B * self.N, d.H, d.V, d.Hq, d.Hkv, d.d, self.node_tokens,
                           w["embed"], w["wq"], w["wk"], w["wv"], self.q, self.k_tree, self.v_tree,
                           self.ws_proxy)
        if d.rope_base > 0.0:
            M.medusa_rope(d.dtype, d.B * self.N, d.Hq, d.Hkv, d.d, self.position_ids, d.rope_base,
                          self.q, self.k_tree)

    def attention(self):
        d, w = self.dims, self.w
        M.medusa_tree_attention(self.plan, d.dtype, d.B, d.Hq, d.Hkv, d.d, d.Lcap, 0.0, self.q,
                                self.k_tree, self.v_tree, w["k_cache"], w["v_cache"],
                                w["prefix_lens"], self.o, self.ws_attn)

    def verifier_out(self):
        d, w = self.dims, self.w
        M.medusa_proxy_out(d.dtype, d.B * self.N, d.H, d.V, d.Hq, d.d, self.node_tokens,
                           w["embed"], self.o, w["wo"], self.node_hidden, self.ws_proxy)

    def verify(self):
        d, w = self.dims, self.w
        if self.typical is not None:
            T, eps, delta = self.typical
            M.medusa_verify_accept_typical(self.plan, d.dtype, d.B, d.H, d.V, self.node_hidden,
                                           w["w_lm"], self.node_tokens, T, eps, delta,
                                           self.node_argmax, self.node_prob, self.node_tau,
                                           self.accept_len, self.accept_nodes, self.accept_tokens,
                                           self.verify_logits, self.ws_verify)
            return
        M.medusa_verify_accept(self.plan, d.dtype, d.B, d.H, d.V, self.node_hidden, w["w_lm"],
                               self.node_tokens, self.node_argmax, self.accept_len,
                               self.accept_nodes, self.accept_tokens, self.verify_logits,
                               self.ws_verify)

    def advance(self, overflow=None):
        """Commit the accepted branches: their tree K/V rows join w["k_cache"]/w["v_cache"]
        after the prefix, w["prefix_lens"] grows, w["h"] becomes the deepest accepted
        node's hidden state and root_ids the bonus token, so the next run() is the next
        round.  The weights dict's cache, lengths and h are updated in place."""
        d, w = self.dims, self.w
        M.medusa_advance(self.plan, d.dtype, d.B, d.H, d.Hkv, d.d, d.Lcap, self.accept_len,
                         self.accept_nodes, self.accept_tokens, self.k_tree, self.v_tree,
                         self.node_hidden, w["k_cache"], w["v_cache"], w["prefix_lens"], w["h"],
                         self.root_ids, overflow)

    # ---- the decode loop's state: everything a round reads that earlier rounds changed
    LOOP_STATE = ("k_cache", "v_cache", "prefix_lens", "h")

    def loop_state(self) -> Dict[str, "object"]:
        """Host copies of the loop state: the KV caches, prefix lengths, last hidden states
        (the weights dict's entries) and the next roots.  With the weights, it is all a
        later round needs."""
        out = {k: self.w[k].detach().cpu().clone() for k in self.LOOP_STATE}
        out["root_ids"] = self.root_ids.detach().cpu().clone()
        return out

    def load_loop_state(self, state: Dict[str, "object"]) -> None:
        """Restore loop_state() into this step's buffers (same shapes); the next run() with
        bootstrap_root=False continues from there."""
        for k in self.LOOP_STATE:
            self.w[k].copy_(state[k])
        self.root_ids.copy_(state["root_ids"])

    def save_loop_state(self, path: str) -> None:
        from safetensors.torch import save_file
        save_file({k: v.contiguous() for k, v in self.loop_state().items()}, path)

    def restore_loop_state(self, path: str) -> None:
        from safetensors.torch import load_file
        self.load_loop_state(load_file(path))

    def decode(self, steps: int, bootstrap_root: bool = True):
        """``steps`` rounds of run() + advance(), all enqueued without a host
        synchronisation.  Returns device tensors: the first roots [B], and per round the
        accepted lengths [steps, B], emitted tokens [steps, B, D+1] (accepted candidates
        then the bonus) and overflow flags [steps, B]."""
        torch = _torch()
        B, D = self.dims.B, self.D
        dev = self.accept_len.device
        lens = torch.empty(steps, B, dtype=torch.int32, device=dev)
        toks = torch.empty(steps, B, D + 1, dtype=torch.int32, device=dev)
        over = torch.empty(steps, B, dtype=torch.int32, device=dev)
        root0 = None
        for i in range(steps):
            self.run(bootstrap_root=bootstrap_root and i == 0, keep_u=False)
            if i == 0:
                root0 = self.root_ids.clone()
            lens[i].copy_(self.accept_len)
            toks[i].copy_(self.accept_tokens)
            self.advance(overflow=over[i])
        return root0, lens, toks, over

    @staticmethod
    def streams(lens, toks):
        """Host copy of each sequence's emitted tokens over the rounds of decode()."""
        lens = lens.cpu().numpy()
        toks = toks.cpu().numpy()
        return [np.concatenate([toks[i, b, : lens[i, b] + 1] for i in range(lens.shape[0])]).astype(np.int64)
                for b in range(lens.shape[1])]

    def run(self, bootstrap_root: bool = False, keep_u: bool = True):
        """Enqueue one whole step.  With bootstrap_root the root token is computed as
        argmax(lm_head(h)); otherwise root_ids holds it (the previous step's bonus)."""
        self.heads(bootstrap_root=bootstrap_root, keep_u=keep_u)
        self.tree()
        self.verifier_in()
        self.attention()
        self.verifier_out()
        self.verify()

    def results(self) -> Dict[str, np.ndarray]:
        """Copy every output back to the host (synchronises)."""
        torch = _torch()

        def host(t):
            if t is None:
                return None
            if t.dtype == torch.bfloat16:
                return t.float().cpu().numpy().astype(np.float64)
            return t.cpu().numpy()

        names = ["topk_ids", "topk_vals", "root_ids", "u", "node_tokens", "position_ids", "q",
                 "k_tree", "v_tree", "o", "node_hidden", "node_argmax", "accept_len",
                 "accept_nodes", "accept_tokens", "head_logits", "verify_logits", "node_prob",
                 "node_tau"]
        out = {n: host(getattr(self, n)) for n in names if n != "u"}
        out["u"] = host(self.u) if getattr(self, "u_written", False) else None
        return out
