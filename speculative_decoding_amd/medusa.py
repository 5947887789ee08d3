"""Thin Python binding of libmedusa: the C-ABI calls under the same names.

Only argument marshalling happens here: tensors are checked for device, dtype and
contiguity and passed as raw pointers together with the current HIP stream.  All
computation runs in the library's HIP kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np

from ._lib import lib

MEDUSA_F32, MEDUSA_BF16 = 0, 1
MEDUSA_MAX_TOPK, MEDUSA_MAX_HEADS, MEDUSA_MAX_NODES = 64, 8, 1024   # limits of include/medusa.h
MEDUSA_NOALLOC_SCRATCH_BYTES = 4194304   # static scratch of medusa_verify_accept_noalloc
DTYPES = {"f32": MEDUSA_F32, "bf16": MEDUSA_BF16}


class MedusaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().medusa_status_string(status).decode()
        extra = ""
        if status == 7:
            extra = f" (hipError {lib().medusa_last_hip_error()})"
        super().__init__(f"{fn}: {msg}{extra}")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MedusaError(fn, status)


def _dt(dt) -> int:
    return DTYPES[dt] if isinstance(dt, str) else int(dt)


def _torch():
    import torch
    return torch


def _ptr(t, dtype=None, name="tensor"):
    """Device pointer of a contiguous CUDA/HIP tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _float_ptr(t, dt, name):
    torch = _torch()
    want = torch.bfloat16 if _dt(dt) == MEDUSA_BF16 else torch.float32
    return _ptr(t, want, name)


def _stream(stream=None):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def _i32_host(seq: Sequence[int]):
    arr = (ctypes.c_int32 * len(seq))(*[int(x) for x in seq])
    return arr


# ------------------------------------------------------------------ plans

class TreePlan:
    """Owner of a medusa_tree_plan (host) and, once uploaded, its device buffer."""

    def __init__(self, handle: ctypes.c_void_p):
        self._h = handle
        self._dev = None

    @property
    def handle(self):
        return self._h

    def info(self):
        n, d, w = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        _check("medusa_tree_plan_info", lib().medusa_tree_plan_info(self._h, ctypes.byref(n),
                                                                     ctypes.byref(d), ctypes.byref(w)))
        return n.value, d.value, w.value

    @property
    def n_nodes(self):
        return self.info()[0]

    @property
    def max_depth(self):
        return self.info()[1]

    def arrays(self):
        n, _, w = self.info()
        parent = np.zeros(n, np.int32)
        depth = np.zeros(n, np.int32)
        rank = np.zeros(n, np.int32)
        mask = np.zeros(n * w, np.uint64)
        P = lambda a, t: a.ctypes.data_as(ctypes.POINTER(t))
        _check("medusa_tree_plan_arrays", lib().medusa_tree_plan_arrays(
            self._h, P(parent, ctypes.c_int32), P(depth, ctypes.c_int32), P(rank, ctypes.c_int32),
            P(mask, ctypes.c_uint64)))
        return parent, depth, rank, mask.reshape(n, w)

    def expected_accept(self, acc: np.ndarray) -> float:
        """Expected accepted length under per-head rank accuracies acc[depth-1][rank]."""
        acc = np.ascontiguousarray(acc, dtype=np.float64)
        out = ctypes.c_double()
        _check("medusa_tree_plan_expected_accept", lib().medusa_tree_plan_expected_accept(
            self._h, acc.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), acc.shape[1],
            acc.shape[0], ctypes.byref(out)))
        return out.value

    def device_bytes(self) -> int:
        return int(lib().medusa_tree_plan_device_bytes(self._h))

    def upload(self, device="cuda", stream=None):
        torch = _torch()
        nbytes = self.device_bytes()
        buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        off = (-buf.data_ptr()) % 256
        _check("medusa_tree_plan_upload", lib().medusa_tree_plan_upload(
            self._h, buf.data_ptr() + off, nbytes, _stream(stream)))
        self._dev = buf
        return self

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            try:
                lib().medusa_tree_plan_destroy(h)
            except Exception:
                pass


def medusa_tree_plan_create(paths: Sequence[Sequence[int]]) -> TreePlan:
    paths = [list(p) for p in paths]
    D = max((len(p) for p in paths), default=1)
    flat = np.full((len(paths), max(D, 1)), -1, np.int32)
    for i, p in enumerate(paths):
        flat[i, : len(p)] = p
    out = ctypes.c_void_p()
    _check("medusa_tree_plan_create", lib().medusa_tree_plan_create(
        flat.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(paths), D, ctypes.byref(out)))
    return TreePlan(out)


def medusa_tree_plan_full(tree_s: Sequence[int]) -> TreePlan:
    out = ctypes.c_void_p()
    _check("medusa_tree_plan_full", lib().medusa_tree_plan_full(
        _i32_host(tree_s), len(tree_s), ctypes.byref(out)))
    return TreePlan(out)


def medusa_tree_plan_from_accuracy(acc: np.ndarray, tree_s: Sequence[int], n_nodes: int) -> TreePlan:
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    out = ctypes.c_void_p()
    _check("medusa_tree_plan_from_accuracy", lib().medusa_tree_plan_from_accuracy(
        acc.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), acc.shape[1], _i32_host(tree_s),
        len(tree_s), int(n_nodes), ctypes.byref(out)))
    return TreePlan(out)


def medusa_tree_plan_expected_accept(plan: TreePlan, acc: np.ndarray) -> float:
    return plan.expected_accept(acc)


# ------------------------------------------------------------------ the four calls

def medusa_heads_workspace(dt, B, H, V, K, s_max) -> int:
    return int(lib().medusa_heads_workspace(_dt(dt), B, H, V, K, s_max))


def medusa_heads_forward(dt, B, H, V, K, hidden, w1, b1, w2, w_lm, s, s_max, topk_ids,
                         topk_vals, root_ids=None, u_out=None, logits=None, ws=None, stream=None):
    torch = _torch()
    st = lib().medusa_heads_forward(
        _dt(dt), B, H, V, K, _float_ptr(hidden, dt, "hidden"), _float_ptr(w1, dt, "w1"),
        _float_ptr(b1, dt, "b1"), _float_ptr(w2, dt, "w2"),
        _float_ptr(w_lm, dt, "w_lm") if w_lm is not None else None, _i32_host(s), s_max,
        _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_vals, torch.float32, "topk_vals"),
        _ptr(root_ids, torch.int32, "root_ids"),
        _float_ptr(u_out, dt, "u_out") if u_out is not None else None,
        _ptr(logits, torch.float32, "logits"), _ptr(ws, None, "ws"),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check("medusa_heads_forward", st)


def medusa_build_tree(plan: TreePlan, B, K, s_max, s, root_ids, topk_ids, prefix_lens,
                      node_tokens, position_ids=None, stream=None):
    torch = _torch()
    st = lib().medusa_build_tree(
        plan.handle, B, K, s_max, _i32_host(s), _ptr(root_ids, torch.int32, "root_ids"),
        _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(prefix_lens, torch.int32, "prefix_lens"),
        _ptr(node_tokens, torch.int32, "node_tokens"),
        _ptr(position_ids, torch.int32, "position_ids"), _stream(stream))
    _check("medusa_build_tree", st)


def medusa_attention_workspace(plan: TreePlan, dt, B, Hq, Hkv, d, Lcap) -> int:
    return int(lib().medusa_attention_workspace(plan.handle, _dt(dt), B, Hq, Hkv, d, Lcap))


def medusa_tree_attention(plan: TreePlan, dt, B, Hq, Hkv, d, Lcap, scale, q, k_tree, v_tree,
                          k_cache, v_cache, prefix_lens, out, ws, stream=None):
    torch = _torch()
    st = lib().medusa_tree_attention(
        plan.handle, _dt(dt), B, Hq, Hkv, d, Lcap, float(scale), _float_ptr(q, dt, "q"),
        _float_ptr(k_tree, dt, "k_tree"), _float_ptr(v_tree, dt, "v_tree"),
        _float_ptr(k_cache, dt, "k_cache"), _float_ptr(v_cache, dt, "v_cache"),
        _ptr(prefix_lens, torch.int32, "prefix_lens"), _float_ptr(out, dt, "out"),
        _ptr(ws, None, "ws"), ws.numel() * ws.element_size() if ws is not None else 0,
        _stream(stream))
    _check("medusa_tree_attention", st)


def medusa_verify_workspace(plan: TreePlan, dt, B, H, V) -> int:
    return int(lib().medusa_verify_workspace(plan.handle, _dt(dt), B, H, V))


def medusa_advance(plan: TreePlan, dt, B, H, Hkv, d, Lcap, accept_len, accept_nodes,
                   accept_tokens, k_tree, v_tree, node_hidden, k_cache, v_cache, prefix_lens,
                   hidden_out, root_out, overflow=None, stream=None):
    torch = _torch()
    st = lib().medusa_advance(
        plan.handle, _dt(dt), B, H, Hkv, d, Lcap, _ptr(accept_len, torch.int32, "accept_len"),
        _ptr(accept_nodes, torch.int32, "accept_nodes"),
        _ptr(accept_tokens, torch.int32, "accept_tokens"), _float_ptr(k_tree, dt, "k_tree"),
        _float_ptr(v_tree, dt, "v_tree"), _float_ptr(node_hidden, dt, "node_hidden"),
        _float_ptr(k_cache, dt, "k_cache"), _float_ptr(v_cache, dt, "v_cache"),
        _ptr(prefix_lens, torch.int32, "prefix_lens"), _float_ptr(hidden_out, dt, "hidden_out"),
        _ptr(root_out, torch.int32, "root_out"), _ptr(overflow, torch.int32, "overflow"),
        _stream(stream))
    _check("medusa_advance", st)


def medusa_verify_accept(plan: TreePlan, dt, B, H, V, node_hidden, w_lm, node_tokens,
                         node_argmax, accept_len, accept_nodes, accept_tokens, logits=None,
                         ws=None, stream=None):
    torch = _torch()
    st = lib().medusa_verify_accept(
        plan.handle, _dt(dt), B, H, V, _float_ptr(node_hidden, dt, "node_hidden"),
        _float_ptr(w_lm, dt, "w_lm"), _ptr(node_tokens, torch.int32, "node_tokens"),
        _ptr(node_argmax, torch.int32, "node_argmax"), _ptr(accept_len, torch.int32, "accept_len"),
        _ptr(accept_nodes, torch.int32, "accept_nodes"),
        _ptr(accept_tokens, torch.int32, "accept_tokens"), _ptr(logits, torch.float32, "logits"),
        _ptr(ws, None, "ws"), ws.numel() * ws.element_size() if ws is not None else 0,
        _stream(stream))
    _check("medusa_verify_accept", st)


def medusa_verify_accept_noalloc(plan: TreePlan, dt, B, H, V, node_hidden, w_lm, node_tokens,
                                 node_argmax, accept_len, accept_nodes, accept_tokens,
                                 logits=None, stream=None):
    torch = _torch()
    st = lib().medusa_verify_accept_noalloc(
        plan.handle, _dt(dt), B, H, V, _float_ptr(node_hidden, dt, "node_hidden"),
        _float_ptr(w_lm, dt, "w_lm"), _ptr(node_tokens, torch.int32, "node_tokens"),
        _ptr(node_argmax, torch.int32, "node_argmax"), _ptr(accept_len, torch.int32, "accept_len"),
        _ptr(accept_nodes, torch.int32, "accept_nodes"),
        _ptr(accept_tokens, torch.int32, "accept_tokens"), _ptr(logits, torch.float32, "logits"),
        _stream(stream))
    _check("medusa_verify_accept_noalloc", st)


def medusa_verify_typical_workspace(plan: TreePlan, dt, B, H, V) -> int:
    return int(lib().medusa_verify_typical_workspace(plan.handle, _dt(dt), B, H, V))


def medusa_verify_accept_typical(plan: TreePlan, dt, B, H, V, node_hidden, w_lm, node_tokens,
                                 temperature, epsilon, delta, node_argmax, node_prob, node_tau,
                                 accept_len, accept_nodes, accept_tokens, logits=None, ws=None,
                                 stream=None):
    torch = _torch()
    st = lib().medusa_verify_accept_typical(
        plan.handle, _dt(dt), B, H, V, _float_ptr(node_hidden, dt, "node_hidden"),
        _float_ptr(w_lm, dt, "w_lm"), _ptr(node_tokens, torch.int32, "node_tokens"),
        float(temperature), float(epsilon), float(delta),
        _ptr(node_argmax, torch.int32, "node_argmax"), _ptr(node_prob, torch.float32, "node_prob"),
        _ptr(node_tau, torch.float32, "node_tau"), _ptr(accept_len, torch.int32, "accept_len"),
        _ptr(accept_nodes, torch.int32, "accept_nodes"),
        _ptr(accept_tokens, torch.int32, "accept_tokens"), _ptr(logits, torch.float32, "logits"),
        _ptr(ws, None, "ws"), ws.numel() * ws.element_size() if ws is not None else 0,
        _stream(stream))
    _check("medusa_verify_accept_typical", st)


def medusa_rope(dt, M, Hq, Hkv, d, positions, base, q, k, stream=None):
    torch = _torch()
    st = lib().medusa_rope(_dt(dt), M, Hq, Hkv, d, _ptr(positions, torch.int32, "positions"),
                           float(base), _float_ptr(q, dt, "q"), _float_ptr(k, dt, "k"),
                           _stream(stream))
    _check("medusa_rope", st)


def medusa_hbm_probe_bytes(nbytes: int) -> int:
    return int(lib().medusa_hbm_probe_bytes(int(nbytes)))


def medusa_hbm_read_probe(buf, sink, stream=None):
    """One streaming read of a device tensor's bytes; sink: a device tensor of >= 4 bytes."""
    st = lib().medusa_hbm_read_probe(_ptr(buf, None, "buf"), buf.numel() * buf.element_size(),
                                     _ptr(sink, None, "sink"), _stream(stream))
    _check("medusa_hbm_read_probe", st)


def medusa_clock_probe(ticks, sink, stream=None):
    """ticks: int64 [2] device tensor (shader clock ticks, 100 MHz ticks); sink: int32 [1]."""
    torch = _torch()
    st = lib().medusa_clock_probe(_ptr(ticks, torch.int64, "ticks"), _ptr(sink, torch.int32, "sink"),
                                  _stream(stream))
    _check("medusa_clock_probe", st)


def medusa_proxy_workspace(dt, M, H, Hq, Hkv, d) -> int:
    return int(lib().medusa_proxy_workspace(_dt(dt), M, H, Hq, Hkv, d))


def medusa_proxy_qkv(dt, M, H, V, Hq, Hkv, d, tokens, embed, wq, wk, wv, q, k, v, ws,
                     stream=None):
    torch = _torch()
    st = lib().medusa_proxy_qkv(
        _dt(dt), M, H, V, Hq, Hkv, d, _ptr(tokens, torch.int32, "tokens"),
        _float_ptr(embed, dt, "embed"), _float_ptr(wq, dt, "wq"), _float_ptr(wk, dt, "wk"),
        _float_ptr(wv, dt, "wv"), _float_ptr(q, dt, "q"), _float_ptr(k, dt, "k"),
        _float_ptr(v, dt, "v"), _ptr(ws, None, "ws"),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check("medusa_proxy_qkv", st)


def medusa_proxy_out(dt, M, H, V, Hq, d, tokens, embed, o, wo, node_hidden, ws, stream=None):
    torch = _torch()
    st = lib().medusa_proxy_out(
        _dt(dt), M, H, V, Hq, d, _ptr(tokens, torch.int32, "tokens"),
        _float_ptr(embed, dt, "embed"), _float_ptr(o, dt, "o"), _float_ptr(wo, dt, "wo"),
        _float_ptr(node_hidden, dt, "node_hidden"), _ptr(ws, None, "ws"),
        ws.numel() * ws.element_size() if ws is not None else 0, _stream(stream))
    _check("medusa_proxy_out", st)


# ------------------------------------------------------------------ profiling

def medusa_profile_enable(on: bool = True) -> None:
    _check("medusa_profile_enable", lib().medusa_profile_enable(1 if on else 0))


def medusa_profile_only(kernel=None) -> None:
    _check("medusa_profile_only", lib().medusa_profile_only(kernel.encode() if kernel else None))


def medusa_profile_reset() -> None:
    _check("medusa_profile_reset", lib().medusa_profile_reset())


def medusa_profile_query(kernel: str):
    ms = ctypes.c_double()
    n = ctypes.c_int()
    _check("medusa_profile_query", lib().medusa_profile_query(kernel.encode(), ctypes.byref(ms),
                                                              ctypes.byref(n)))
    return ms.value, n.value
