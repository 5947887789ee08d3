"""GPU parity of medusa_rope (rotary positions on the verifier's q and k, in place) against
the oracle's rope on the same stored values, at positions up to the largest cache the
library accepts (2^20), for both storage types and head sizes 8, 64 and 128; position 0
leaves every value's bits unchanged."""
import numpy as np
import pytest

import oracle
from synth import integers, normal_bf16
from tests.gpu_util import close, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from speculative_decoding_amd import lib
    lib()
    return torch.device("cuda:0")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("M,Hq,Hkv,d,pmax", [(5, 3, 1, 8, 40), (64, 32, 8, 128, 1 << 20),
                                             (17, 4, 2, 64, 70000)])
def test_rope_against_oracle(dev, dt, M, Hq, Hkv, d, pmax):
    import torch
    from speculative_decoding_amd import medusa as M_
    say(f"[rope {dt} M={M} Hq={Hq} Hkv={Hkv} d={d} positions < {pmax}]")
    seed, base = 21, 10000.0
    q = normal_bf16(seed, f"rope{d}/q", (M, Hq, d), 1.0)
    k = normal_bf16(seed, f"rope{d}/k", (M, Hkv, d), 1.0)
    pos = integers(seed, f"rope{d}/pos", 0, pmax, (M,)).astype(np.int32)
    pos[0] = 0
    qf, kf = oracle.as_f64(q, "bf16"), oracle.as_f64(k, "bf16")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    tq = torch.from_numpy(qf.astype(np.float32)).to(dev).to(tdt).contiguous()
    tk = torch.from_numpy(kf.astype(np.float32)).to(dev).to(tdt).contiguous()
    q0, k0 = tq.clone(), tk.clone()
    tpos = torch.from_numpy(pos).to(dev)
    M_.medusa_rope(dt, M, Hq, Hkv, d, tpos, base, tq, tk)
    torch.cuda.synchronize()
    want_q = oracle.round_act(oracle.rope(qf, pos, base), dt)
    want_k = oracle.round_act(oracle.rope(kf, pos, base), dt)
    close("q", tq.float().cpu().numpy(), want_q)
    close("k", tk.float().cpu().numpy(), want_k)
    assert torch.equal(tq[0], q0[0]) and torch.equal(tk[0], k0[0]), "position 0 changed a value"
    if dt == "f32":
        # fp32 storage: the rotation itself is within a few fp32 ulps of fp64
        np.testing.assert_allclose(tq.cpu().numpy(), oracle.rope(qf, pos, base), rtol=0, atol=2e-5)
