"""Workload shapes for the Medusa decode step.

Each configuration fixes the shapes, the storage dtype and the distribution
every tensor is drawn from.  Weights are row-major ``[out, in]``, the
``nn.Linear`` convention of the PyTorch example on the Ultralytics glossary
page (section "Comment les têtes prédisent les tokens suivants").  ``N(0, s)``
means a normal with standard deviation ``s``.

The pages give only one concrete shape, the worked example with hidden size
256, vocabulary 1000 and three heads (same section).  The other shapes are
model-like workloads: an 8B-class decoder (hidden 4096, Llama-3 vocabulary
128256, grouped-query attention 32/8), a 7B-class decoder with a 32000
vocabulary, a 70B-class decoder (hidden 8192) at batch 8, and a dense-tree
variant of the 8B shape.  The sparse 64-node tree and the dense 256-node tree
follow the glossary page's remark (section "Attention arborescente et
acceptation") that a 64-node sparse tree built from the most accurate
combinations beats a 256-node dense tree.

Two further, smaller bf16 shapes exist only for parity tests: they span several
kernel tiles, end in a ragged tail and include a zero-length prefix, while the
CPU oracle still finishes in seconds.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    B: int                      # sequences
    H: int                      # hidden size
    V: int                      # vocabulary
    K: int                      # Medusa heads
    s: Tuple[int, ...]          # top-k kept per head (len K)
    tree: str                   # "full": Cartesian product of tree_s; "sparse": top n_nodes-1 by accuracy
    tree_s: Tuple[int, ...]     # per-depth branching used to enumerate candidate rank tuples
    n_nodes: int                # tree nodes including the root
    Hq: int
    Hkv: int
    d: int
    L: int = 0                  # prefix length when every sequence has the same one
    L_range: Optional[Tuple[int, int]] = None   # inclusive uniform range per sequence
    lens: Optional[Tuple[int, ...]] = None      # explicit per-sequence prefix lengths
    Lcap: int = 0               # KV-cache rows allocated per sequence
    dtype: str = "bf16"         # storage/activation dtype: "bf16" or "f32"
    sigma_lm: float = 0.0       # lm_head rows
    sigma_w1: float = 0.0       # head FF weight
    b1_zero: bool = False       # head FF bias all zero
    sigma_b1: float = 0.0
    w2_copy_lm: bool = False    # head projections start as a copy of lm_head
    sigma_w2: float = 0.0
    sigma_proxy: float = 0.0    # Wq, Wk, Wv, Wo of the one-layer verifier
    sigma_embed: float = 1.0    # token embedding table E
    sigma_h: float = 1.0        # last hidden state
    sigma_kv: float = 1.0       # cached K/V prefix
    rope_base: float = 0.0      # rotary position embedding base of the verifier (0: none)
    note: str = field(default="", compare=False)

    @property
    def s_max(self) -> int:
        return max(self.s)

    @property
    def depth(self) -> int:
        return len(self.tree_s)

    def prefix_lens_fixed(self) -> Optional[Tuple[int, ...]]:
        if self.lens is not None:
            return tuple(self.lens)
        if self.L_range is None:
            return (self.L,) * self.B
        return None


def _inv_sqrt(n: int) -> float:
    return 1.0 / float(n) ** 0.5


CONFIGS = {
    # Worked-example shape of the glossary page: hidden 256, vocab 1000, 3 heads,
    # FF init N(0, 0.02) with zero bias, projections copied from lm_head; fp32.
    "tiny": Config(
        name="tiny", B=1, H=256, V=1000, K=3, s=(2, 3, 3), tree="full", tree_s=(2, 3),
        n_nodes=9, Hq=4, Hkv=4, d=64, L=32, Lcap=32, dtype="f32",
        sigma_lm=_inv_sqrt(256), sigma_w1=0.02, b1_zero=True, w2_copy_lm=True,
        sigma_proxy=_inv_sqrt(256)),
    # 7B-class decoder, 32000 vocabulary, multi-head attention, 5 heads.
    "mid": Config(
        name="mid", B=1, H=4096, V=32000, K=5, s=(10, 5, 4, 3, 2), tree="sparse",
        tree_s=(10, 5, 4, 3, 2), n_nodes=64, Hq=32, Hkv=32, d=128, L=1024, Lcap=1024,
        sigma_lm=_inv_sqrt(4096), sigma_w1=_inv_sqrt(4096), sigma_b1=_inv_sqrt(4096),
        sigma_w2=_inv_sqrt(4096), sigma_proxy=_inv_sqrt(4096)),
    # 8B-class decoder (Llama-3 vocabulary, GQA 32/8), 4 heads, sparse 64-node tree.
    "8b": Config(
        name="8b", B=1, H=4096, V=128256, K=4, s=(10, 5, 4, 3), tree="sparse",
        tree_s=(10, 5, 4, 3), n_nodes=64, Hq=32, Hkv=8, d=128, L=4096, Lcap=4096,
        sigma_lm=_inv_sqrt(4096), sigma_w1=_inv_sqrt(4096), sigma_b1=_inv_sqrt(4096),
        sigma_w2=_inv_sqrt(4096), sigma_proxy=_inv_sqrt(4096)),
    # The 8B shape with the full Cartesian tree 1 + 3 + 12 + 48 + 192 = 256 nodes,
    # prefix 8192.
    "dense": Config(
        name="dense", B=1, H=4096, V=128256, K=4, s=(3, 4, 4, 4), tree="full",
        tree_s=(3, 4, 4, 4), n_nodes=256, Hq=32, Hkv=8, d=128, L=8192, Lcap=8192,
        sigma_lm=_inv_sqrt(4096), sigma_w1=_inv_sqrt(4096), sigma_b1=_inv_sqrt(4096),
        sigma_w2=_inv_sqrt(4096), sigma_proxy=_inv_sqrt(4096)),
    # 70B-class decoder at batch 8, ragged prefixes uniform in [512, 8192].
    "batched70b": Config(
        name="batched70b", B=8, H=8192, V=32000, K=5, s=(10, 5, 4, 3, 2), tree="sparse",
        tree_s=(10, 5, 4, 3, 2), n_nodes=64, Hq=64, Hkv=8, d=128, L_range=(512, 8192),
        Lcap=8192,
        sigma_lm=_inv_sqrt(8192), sigma_w1=_inv_sqrt(8192), sigma_b1=_inv_sqrt(8192),
        sigma_w2=_inv_sqrt(8192), sigma_proxy=_inv_sqrt(8192)),
    # Parity-test shapes: several tiles, ragged vocabulary (prime), ragged prefixes.
    "small": Config(
        name="small", B=1, H=512, V=5003, K=4, s=(10, 5, 4, 3), tree="sparse",
        tree_s=(10, 5, 4, 3), n_nodes=64, Hq=8, Hkv=2, d=128, L=300, Lcap=320,
        sigma_lm=_inv_sqrt(512), sigma_w1=_inv_sqrt(512), sigma_b1=_inv_sqrt(512),
        sigma_w2=_inv_sqrt(512), sigma_proxy=_inv_sqrt(512)),
    "small_batched": Config(
        name="small_batched", B=3, H=512, V=3001, K=3, s=(4, 3, 2), tree="sparse",
        tree_s=(4, 3, 2), n_nodes=16, Hq=4, Hkv=1, d=64, lens=(0, 129, 300), Lcap=300,
        sigma_lm=_inv_sqrt(512), sigma_w1=_inv_sqrt(512), sigma_b1=_inv_sqrt(512),
        sigma_w2=_inv_sqrt(512), sigma_proxy=_inv_sqrt(512)),
    # a full 4x4x4 tree (85 nodes) for two sequences: 170 verified rows, more than one
    # 64-row block of the lm_head kernels, the last one ragged
    "small_dense": Config(
        name="small_dense", B=2, H=512, V=2003, K=3, s=(4, 4, 4), tree="full",
        tree_s=(4, 4, 4), n_nodes=85, Hq=4, Hkv=2, d=64, lens=(100, 257), Lcap=260,
        sigma_lm=_inv_sqrt(512), sigma_w1=_inv_sqrt(512), sigma_b1=_inv_sqrt(512),
        sigma_w2=_inv_sqrt(512), sigma_proxy=_inv_sqrt(512)),
    # node budgets at the small shape: the root alone (no candidates, one verified row per
    # sequence) and a wide 341-node tree (several 64-row blocks with a ragged last one)
    "small_n1": Config(
        name="small_n1", B=1, H=512, V=5003, K=4, s=(10, 5, 4, 3), tree="sparse",
        tree_s=(10, 5, 4, 3), n_nodes=1, Hq=8, Hkv=2, d=128, L=300, Lcap=320,
        sigma_lm=_inv_sqrt(512), sigma_w1=_inv_sqrt(512), sigma_b1=_inv_sqrt(512),
        sigma_w2=_inv_sqrt(512), sigma_proxy=_inv_sqrt(512)),
    "small_n341": Config(
        name="small_n341", B=1, H=512, V=5003, K=4, s=(10, 5, 4, 3), tree="sparse",
        tree_s=(10, 5, 4, 3), n_nodes=341, Hq=8, Hkv=2, d=128, L=300, Lcap=320,
        sigma_lm=_inv_sqrt(512), sigma_w1=_inv_sqrt(512), sigma_b1=_inv_sqrt(512),
        sigma_w2=_inv_sqrt(512), sigma_proxy=_inv_sqrt(512)),
    # the library's limits at a small shape: 8 heads, top-64 on the first, a 1024-node
    # tree (several mask words, 2048 verified rows), an empty and a ragged prefix
    "small_max": Config(
        name="small_max", B=2, H=512, V=3001, K=8, s=(64, 4, 3, 2, 2, 2, 2, 2), tree="sparse",
        tree_s=(64, 4, 3, 2, 2, 2, 2, 2), n_nodes=1024, Hq=4, Hkv=1, d=64, lens=(0, 201),
        Lcap=256,
        sigma_lm=_inv_sqrt(512), sigma_w1=_inv_sqrt(512), sigma_b1=_inv_sqrt(512),
        sigma_w2=_inv_sqrt(512), sigma_proxy=_inv_sqrt(512)),
    # the largest batch the heads accept (64 sequences), ragged prefixes from empty to full
    "small_b64": Config(
        name="small_b64", B=64, H=256, V=1000, K=3, s=(2, 3, 3), tree="full", tree_s=(2, 3),
        n_nodes=9, Hq=4, Hkv=2, d=64, L_range=(0, 64), Lcap=64,
        sigma_lm=_inv_sqrt(256), sigma_w1=_inv_sqrt(256), sigma_b1=_inv_sqrt(256),
        sigma_w2=_inv_sqrt(256), sigma_proxy=_inv_sqrt(256)),
    # the verifier with rotary positions (base 10000): ragged prefixes including an empty
    # one, and a loop case whose rounds move the positions on
    "small_rope": Config(
        name="small_rope", B=3, H=512, V=3001, K=3, s=(4, 3, 2), tree="sparse",
        tree_s=(4, 3, 2), n_nodes=16, Hq=4, Hkv=1, d=64, lens=(0, 129, 300), Lcap=300,
        sigma_lm=_inv_sqrt(512), sigma_w1=_inv_sqrt(512), sigma_b1=_inv_sqrt(512),
        sigma_w2=_inv_sqrt(512), sigma_proxy=_inv_sqrt(512), rope_base=10000.0),
    "small_rope_loop": Config(
        name="small_rope_loop", B=2, H=512, V=3001, K=3, s=(4, 3, 2), tree="sparse",
        tree_s=(4, 3, 2), n_nodes=16, Hq=4, Hkv=2, d=128, lens=(40, 97), Lcap=160,
        sigma_lm=_inv_sqrt(512), sigma_w1=_inv_sqrt(512), sigma_b1=_inv_sqrt(512),
        sigma_w2=_inv_sqrt(512), sigma_proxy=_inv_sqrt(512), rope_base=10000.0),
    # decode-loop cases: room in the KV cache for several rounds of accepted branches
    "tiny_loop": Config(
        name="tiny_loop", B=1, H=256, V=1000, K=3, s=(2, 3, 3), tree="full", tree_s=(2, 3),
        n_nodes=9, Hq=4, Hkv=4, d=64, L=32, Lcap=64, dtype="f32",
        sigma_lm=_inv_sqrt(256), sigma_w1=_inv_sqrt(256), sigma_b1=_inv_sqrt(256),
        sigma_w2=_inv_sqrt(256), sigma_proxy=_inv_sqrt(256)),
    "small_loop": Config(
        name="small_loop", B=2, H=512, V=3001, K=3, s=(4, 3, 2), tree="sparse",
        tree_s=(4, 3, 2), n_nodes=16, Hq=4, Hkv=2, d=64, lens=(40, 97), Lcap=160,
        sigma_lm=_inv_sqrt(512), sigma_w1=_inv_sqrt(512), sigma_b1=_inv_sqrt(512),
        sigma_w2=_inv_sqrt(512), sigma_proxy=_inv_sqrt(512)),
}


def get_config(name: str) -> Config:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown config {name!r}; known: {sorted(CONFIGS)}") from None
