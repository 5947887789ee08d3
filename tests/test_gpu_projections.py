"""GPU parity of the verifier's two projections (medusa_proxy_qkv, medusa_proxy_out) on
their own, against the oracle's proxy_qkv / proxy_out.

In a whole step the output projection is a small correction on top of the embedding
residual, so a step-level check cannot see it go wrong; here the inputs make every term
count (one case has a zero residual, so node_hidden is the projection alone).  The shapes
cover each kernel choice: one workgroup per CU (64 rows, 8B-class sizes), row tiles that
run across the q/k/v boundary, fewer than 64 rows, at most 16 (split-contraction store:
the row-contiguous form when the contraction is a multiple of 256, the operand-layout
form otherwise), k/v widths that are not a multiple of 32 (single-wave kernel), 128 rows
or more (256 x 256 tiles in contraction slices, also with widths that end in a partial
tile and row counts that end in a partial block), and a contraction that is not a
multiple of 64 at 200 rows (split-contraction store over several row blocks)."""
import numpy as np
import pytest

import oracle
from synth import integers, normal_bf16
from tests.gpu_util import close, say

pytestmark = pytest.mark.gpu

# name: (M, H, V, Hq, Hkv, d)
CASES = {
    "8b_shape": (64, 4096, 1000, 32, 8, 128),
    "small": (64, 512, 300, 4, 1, 64),
    "rows48": (48, 512, 300, 4, 1, 64),
    "rows16": (16, 512, 300, 4, 1, 64),
    "rows130": (130, 512, 300, 4, 1, 64),
    "qkv_boundary": (40, 1024, 500, 6, 2, 80),
    "kv_width16": (64, 512, 300, 6, 1, 16),
    "rows512": (512, 512, 300, 4, 1, 64),
    "rows400_ragged": (400, 1024, 500, 6, 1, 80),
    "rows8": (8, 512, 300, 4, 1, 64),
    "rows8_h320": (8, 320, 300, 4, 1, 64),
    "rows200_h544": (200, 544, 300, 4, 1, 64),
}


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from speculative_decoding_amd import lib
    lib()
    return torch.device("cuda:0")


def _dev(a, device):
    from speculative_decoding_amd.step import host_to_device
    return host_to_device(a, "bf16", device)


def _host(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("residual", ["embed", "zero"])
def test_projections(dev, name, residual):
    import torch
    from speculative_decoding_amd import medusa as M
    Mr, H, V, Hq, Hkv, d = CASES[name]
    say(f"[projections {name} residual={residual}]")
    seed = 11
    emb = normal_bf16(seed, f"{name}/embed", (V, H), 1.0)
    if residual == "zero":
        emb_out = np.zeros_like(emb)
    else:
        emb_out = emb
    wq = normal_bf16(seed, f"{name}/wq", (Hq * d, H), H ** -0.5)
    wk = normal_bf16(seed, f"{name}/wk", (Hkv * d, H), H ** -0.5)
    wv = normal_bf16(seed, f"{name}/wv", (Hkv * d, H), H ** -0.5)
    wo = normal_bf16(seed, f"{name}/wo", (H, Hq * d), (Hq * d) ** -0.5)
    o = normal_bf16(seed, f"{name}/o", (Mr, Hq, d), 1.0)
    tokens = integers(seed, f"{name}/tokens", 0, V, (1, Mr))

    x_ref, q_ref, k_ref, v_ref = oracle.proxy_qkv(tokens, emb, wq, wk, wv, Hq, Hkv, d, "bf16")
    x_out = oracle.as_f64(emb_out[tokens.reshape(-1)], "bf16").reshape(1, Mr, H)
    nh_ref = oracle.proxy_out(x_out, oracle.as_f64(o, "bf16").reshape(1, Mr, Hq, d), wo, "bf16")

    bf = torch.bfloat16
    t_tok = torch.from_numpy(tokens.reshape(-1).copy()).to(dev)
    t_emb, t_emb_out = _dev(emb, dev), _dev(emb_out, dev)
    t_wq, t_wk, t_wv, t_wo, t_o = (_dev(a, dev) for a in (wq, wk, wv, wo, o))
    q = torch.empty(Mr, Hq * d, dtype=bf, device=dev)
    k = torch.empty(Mr, Hkv * d, dtype=bf, device=dev)
    v = torch.empty(Mr, Hkv * d, dtype=bf, device=dev)
    nh = torch.empty(Mr, H, dtype=bf, device=dev)
    ws = torch.empty(M.medusa_proxy_workspace("bf16", Mr, H, Hq, Hkv, d), dtype=torch.uint8, device=dev)
    outs = []
    for _ in range(2):      # the second call reuses the workspace: results must not change
        M.medusa_proxy_qkv("bf16", Mr, H, V, Hq, Hkv, d, t_tok, t_emb, t_wq, t_wk, t_wv, q, k, v, ws)
        M.medusa_proxy_out("bf16", Mr, H, V, Hq, d, t_tok, t_emb_out, t_o, t_wo, nh, ws)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (q, k, v, nh)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{name}: second call differs"
    close(f"{name} q", _host(q).reshape(q_ref.shape), q_ref)
    close(f"{name} k", _host(k).reshape(k_ref.shape), k_ref)
    close(f"{name} v", _host(v).reshape(v_ref.shape), v_ref)
    close(f"{name} node_hidden", _host(nh).reshape(nh_ref.shape), nh_ref)
