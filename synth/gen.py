"""Seeded tensor generator.

Every tensor comes from its own numpy PCG64 stream, keyed by
``(seed, config name, tensor name[, chunk])`` through ``SeedSequence``, so a
given ``(config, seed)`` always yields the same bytes, independent of the
number of threads used to draw them.  Values are drawn as float32 normals times
the configured standard deviation and, for bf16 workloads, rounded to bf16 with
round-to-nearest-even and kept as raw ``uint16`` bit patterns.

A patch (a list of row swaps and bf16 bit increments, written by the planting
script that lives with the tests) can be applied on top; applying one is pure
data movement.
"""
from __future__ import annotations

import json
import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

from .configs import Config, get_config

_ROWS_PER_CHUNK = 4096


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    r = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _key(seed: int, cfg_name: str, tensor: str, *extra: int):
    return [int(seed) & 0xFFFFFFFF, zlib.crc32(cfg_name.encode()), zlib.crc32(tensor.encode()),
            *[int(e) & 0xFFFFFFFF for e in extra]]


def _rng(seed: int, cfg_name: str, tensor: str, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(_key(seed, cfg_name, tensor, *extra))))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_matrix(seed: int, cfg: Config, tensor: str, rows: int, cols: int, sigma: float,
                   bf16: bool, pool: Optional[ThreadPoolExecutor]) -> np.ndarray:
    """[rows, cols] N(0, sigma), drawn chunk by chunk (4096 rows per chunk)."""
    out = np.empty((rows, cols), dtype=np.uint16 if bf16 else np.float32)
    n_chunks = (rows + _ROWS_PER_CHUNK - 1) // _ROWS_PER_CHUNK

    def work(c: int) -> None:
        r0 = c * _ROWS_PER_CHUNK
        r1 = min(rows, r0 + _ROWS_PER_CHUNK)
        g = _rng(seed, cfg.name, tensor, c)
        buf = g.standard_normal((r1 - r0, cols), dtype=np.float32)
        buf *= np.float32(sigma)
        out[r0:r1] = f32_to_bf16_bits(buf) if bf16 else buf

    if pool is None or n_chunks == 1:
        for c in range(n_chunks):
            work(c)
    else:
        list(pool.map(work, range(n_chunks)))
    return out


def normal_bf16(seed: int, tag: str, shape, sigma: float) -> np.ndarray:
    """A standalone seeded N(0, sigma) tensor of any shape as bf16 bit patterns (uint16),
    for unit-level parity cases that need no full configuration."""
    g = _rng(seed, "standalone", tag)
    buf = g.standard_normal(tuple(shape), dtype=np.float32)
    buf *= np.float32(sigma)
    return f32_to_bf16_bits(buf)


def integers(seed: int, tag: str, low: int, high: int, shape) -> np.ndarray:
    """A standalone seeded uniform integer tensor in [low, high) (int32)."""
    return _rng(seed, "standalone", tag).integers(low, high, size=tuple(shape)).astype(np.int32)


@dataclass
class Inputs:
    """All tensors of one Medusa decode step, as produced by the generator.

    Floating tensors are ``uint16`` bf16 bit patterns when ``dtype == "bf16"``
    and ``float32`` otherwise.
    """
    cfg: Config
    seed: int
    attempt: int
    dtype: str
    h: np.ndarray            # [B, H]
    w_lm: np.ndarray         # [V, H]
    w1: np.ndarray           # [K, H, H]
    b1: np.ndarray           # [K, H]
    w2: np.ndarray           # [K, V, H]
    embed: np.ndarray        # [V, H]
    wq: np.ndarray           # [Hq*d, H]
    wk: np.ndarray           # [Hkv*d, H]
    wv: np.ndarray           # [Hkv*d, H]
    wo: np.ndarray           # [H, Hq*d]
    k_cache: np.ndarray      # [B, Lcap, Hkv, d]
    v_cache: np.ndarray      # [B, Lcap, Hkv, d]
    prefix_lens: np.ndarray  # [B] int32
    acc: np.ndarray          # [K, s_max] float64, per-head rank accuracies (descending)
    plant_rank: np.ndarray   # [B, K] int32, planted rank of the greedy token per head, -1 = miss
    zero_init: bool = False
    patch: Optional[dict] = field(default=None, repr=False)

    def tensors(self) -> Dict[str, np.ndarray]:
        return {k: getattr(self, k) for k in
                ("h", "w_lm", "w1", "b1", "w2", "embed", "wq", "wk", "wv", "wo",
                 "k_cache", "v_cache")}


def accuracy_table(cfg: Config, seed: int) -> np.ndarray:
    """Synthetic per-head rank accuracies acc[k][i] (probability that head k's
    rank-i candidate is the greedy token), falling with depth and rank:
    0.8 * 0.8**k * 0.6 * 0.4**i * U(0.9, 1.1) for 0-based head k, re-sorted
    descending within each head.  Entries beyond s_k are zero."""
    g = _rng(seed, cfg.name, "acc")
    acc = np.zeros((cfg.K, cfg.s_max), dtype=np.float64)
    for k in range(cfg.K):
        sk = cfg.s[k]
        base = 0.8 * (0.8 ** k) * 0.6 * (0.4 ** np.arange(sk))
        jitter = g.uniform(0.9, 1.1, size=sk)
        acc[k, :sk] = np.sort(base * jitter)[::-1]
    return acc


def _plant_ranks(cfg: Config, seed: int, acc: np.ndarray) -> np.ndarray:
    """Draw, per sequence and head, the rank at which the greedy token is to be
    planted: categorical over acc[k][0..s_k) plus a miss with the remaining mass."""
    g = _rng(seed, cfg.name, "plant_rank")
    out = np.full((cfg.B, cfg.K), -1, dtype=np.int32)
    for b in range(cfg.B):
        for k in range(cfg.K):
            sk = cfg.s[k]
            p = acc[k, :sk]
            x = g.uniform()
            c = np.cumsum(p)
            idx = int(np.searchsorted(c, x, side="right"))
            out[b, k] = idx if idx < sk else -1
    return out


def _prefix_lens(cfg: Config, seed: int) -> np.ndarray:
    fixed = cfg.prefix_lens_fixed()
    if fixed is not None:
        return np.asarray(fixed, dtype=np.int32)
    lo, hi = cfg.L_range
    g = _rng(seed, cfg.name, "prefix_lens")
    return g.integers(lo, hi + 1, size=cfg.B).astype(np.int32)


def make_inputs(cfg, seed: int = 0, attempt: Optional[int] = None, patch=None,
                zero_init: bool = False, threads: Optional[int] = None) -> Inputs:
    """Draw every tensor for ``(cfg, seed)``.

    ``attempt`` re-draws only the last hidden state ``h`` (stream key gets the
    attempt number); by default it is taken from the patch, else 0.  ``patch``
    is a dict or a path to a JSON patch file.  ``zero_init`` gives the heads a
    zero FF layer and projections equal to lm_head (no patch allowed then).
    """
    if isinstance(cfg, str):
        cfg = get_config(cfg)
    if isinstance(patch, (str, os.PathLike)):
        with open(patch) as f:
            patch = json.load(f)
    if patch is not None:
        if patch.get("config") != cfg.name or int(patch.get("seed", -1)) != int(seed):
            raise ValueError("patch was written for a different (config, seed)")
        if zero_init:
            raise ValueError("a zero-init draw takes no patch")
        if attempt is None:
            attempt = int(patch.get("h_attempt", 0))
    if attempt is None:
        attempt = 0
    bf16 = cfg.dtype == "bf16"
    n_thr = threads if threads is not None else _threads()
    pool = ThreadPoolExecutor(n_thr) if n_thr > 1 else None
    try:
        B, H, V, K = cfg.B, cfg.H, cfg.V, cfg.K
        qd, kvd = cfg.Hq * cfg.d, cfg.Hkv * cfg.d
        mat = lambda name, r, c, s: _normal_matrix(seed, cfg, name, r, c, s, bf16, pool)
        w_lm = mat("w_lm", V, H, cfg.sigma_lm)
        embed = mat("embed", V, H, cfg.sigma_embed)
        if zero_init:
            w1 = np.zeros((K, H, H), dtype=w_lm.dtype)
            b1 = np.zeros((K, H), dtype=w_lm.dtype)
            w2 = np.stack([w_lm] * K)
        else:
            w1 = np.stack([mat(f"w1.{k}", H, H, cfg.sigma_w1) for k in range(K)])
            if cfg.b1_zero:
                b1 = np.zeros((K, H), dtype=w_lm.dtype)
            else:
                b1 = mat("b1", K, H, cfg.sigma_b1)
            if cfg.w2_copy_lm:
                w2 = np.stack([w_lm] * K)
            else:
                w2 = np.empty((K, V, H), dtype=w_lm.dtype)
                for k in range(K):
                    w2[k] = mat(f"w2.{k}", V, H, cfg.sigma_w2)
        wq = mat("wq", qd, H, cfg.sigma_proxy)
        wk = mat("wk", kvd, H, cfg.sigma_proxy)
        wv = mat("wv", kvd, H, cfg.sigma_proxy)
        wo = mat("wo", H, qd, cfg.sigma_proxy)
        kv_rows = B * cfg.Lcap
        k_cache = mat("k_cache", kv_rows, kvd, cfg.sigma_kv).reshape(B, cfg.Lcap, cfg.Hkv, cfg.d)
        v_cache = mat("v_cache", kv_rows, kvd, cfg.sigma_kv).reshape(B, cfg.Lcap, cfg.Hkv, cfg.d)
        h = _normal_matrix(seed, cfg, f"h.attempt{attempt}", B, H, cfg.sigma_h, bf16, None)
    finally:
        if pool is not None:
            pool.shutdown()
    acc = accuracy_table(cfg, seed)
    inp = Inputs(cfg=cfg, seed=int(seed), attempt=int(attempt), dtype=cfg.dtype, h=h, w_lm=w_lm,
                 w1=w1, b1=b1, w2=w2, embed=embed, wq=wq, wk=wk, wv=wv, wo=wo,
                 k_cache=k_cache, v_cache=v_cache, prefix_lens=_prefix_lens(cfg, seed), acc=acc,
                 plant_rank=_plant_ranks(cfg, seed, acc), zero_init=zero_init)
    if patch is not None:
        if "plant_rank" in patch:
            # a patch written for a chosen acceptance pattern names the ranks it planted
            pr = np.asarray(patch["plant_rank"], dtype=np.int32)
            if pr.shape != inp.plant_rank.shape:
                raise ValueError(f"patch plant_rank has shape {pr.shape}, want "
                                 f"{inp.plant_rank.shape}")
            inp.plant_rank = pr
        apply_patch(inp, patch)
    return inp


# --------------------------------------------------------------------------- patches

def _target(inp: Inputs, op: dict) -> np.ndarray:
    name = op["tensor"]
    if name == "w2":
        return inp.w2[int(op["head"])]
    if name in ("w_lm", "embed"):
        return getattr(inp, name)
    raise ValueError(f"patch op on unsupported tensor {name!r}")


def apply_patch(inp: Inputs, patch: dict) -> None:
    """Apply a patch in order.  Ops:

    * ``swap_rows``: exchange rows ``a`` and ``b`` of the target matrix.
    * ``add_bits``:  add small signed integers to the bf16 bit patterns of
      row ``row`` at columns ``cols`` (moves those weights by whole ulps).
    * ``set_row``:   replace a float32 row (fp32 workloads only) with the
      listed values.
    """
    for op in patch.get("ops", []):
        kind = op["op"]
        m = _target(inp, op)
        if kind == "swap_rows":
            a, b = int(op["a"]), int(op["b"])
            tmp = m[a].copy()
            m[a] = m[b]
            m[b] = tmp
        elif kind == "add_bits":
            if m.dtype != np.uint16:
                raise ValueError("add_bits needs a bf16 tensor")
            r = int(op["row"])
            cols = np.asarray(op["cols"], dtype=np.int64)
            delta = np.asarray(op["delta"], dtype=np.int32)
            v = m[r, cols].astype(np.int32) + delta
            if np.any(v < 0) or np.any(v > 0xFFFF):
                raise ValueError("add_bits leaves the uint16 range")
            m[r, cols] = v.astype(np.uint16)
        elif kind == "set_row":
            if m.dtype != np.float32:
                raise ValueError("set_row needs an fp32 tensor")
            m[int(op["row"])] = np.asarray(op["values"], dtype=np.float32)
        else:
            raise ValueError(f"unknown patch op {kind!r}")
    inp.patch = patch
