"""GPU parity of the fused route + MXFP8 activation quantisation
(moe_route_quant_local): the routing outputs as moe_route_local's, and the
E4M3 codes and E8M0 scales bit-exact against the oracle's mxfp8_quantize.
Decode sizes run as one launch; larger T take the separate quantisation
launch."""
import numpy as np
import pytest
import torch

import moe_expert_routing_amd as M
import oracle as O
import workloads as W
from gpu_util import assert_parity, assert_workspace_zero, oracle_case, say, to_dev

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def _hidden_bits(T, H, seed):
    """bf16 bit patterns ~ N(0,1) with blocks that reach every branch: all
    zeros, saturation (values far above the block's other values), tiny
    values (subnormal E4M3 codes and flush to zero), bf16 subnormals,
    signed zeros, exact ties of the E4M3 rounding."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    if H >= 256:
        for t in range(T):
            k = t % 8
            b = slice(32 * k, 32 * k + 32)
            if k == 0:
                x[t, b] = 0.0
            elif k == 1:
                x[t, b] *= 1e-3
                x[t, 32 * k] = 3.9   # amax 3.9: others near 2^-9 * 2^-7 scale
            elif k == 2:
                x[t, b] = np.float32(2.0 ** -130) * np.arange(32)   # bf16 subnormals
            elif k == 3:
                x[t, b] = -0.0
                x[t, 32 * k + 5] = 1.0
            elif k == 4:
                # 1 + 1/16 and 1 + 3/16 under a scale of 1 (amax 256): ties
                x[t, b] = np.float32(1.0625)
                x[t, 32 * k + 1] = np.float32(1.1875)
                x[t, 32 * k + 2] = np.float32(256.0)
            elif k == 5:
                x[t, b] = np.float32(-3e38)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    return bits


CASES = [
    ("tiny8", lambda: W.tiny_global(8), 7168),
    ("local16", lambda: W.decode_local(16), 7168),
    ("sweep64", lambda: W.decode_sweep(64, 5), 7168),
    ("one_token", lambda: W.random_case(1, seed=3, off=0, cnt=112), 512),
    ("ragged100", lambda: W.random_case(100, seed=4, off=448, cnt=112), 512),
    ("t1000", lambda: W.random_case(1000, seed=5), 1024),
    ("h32", lambda: W.random_case(5, seed=6, off=112, cnt=112), 32),      # one scale block per row
    ("h96", lambda: W.random_case(64, seed=7), 96),                       # three blocks, 12 chunks
    ("t65", lambda: W.random_case(65, seed=8, off=784, cnt=112), 7168),   # first size past one launch
]


@pytest.mark.parametrize("name,make,H", CASES, ids=[c[0] for c in CASES])
def test_route_quant_matches_oracle(name, make, H):
    c = make()
    T = c.logits.shape[0]
    say(f"case route+quant {name} T={T} H={H}")
    bits = _hidden_bits(T, H, seed=T + H)
    out = M.route_quant_local(to_dev(c.logits), to_dev(c.bias), to_dev(bits.view(np.int16)),
                              c.off, c.cnt)
    torch.cuda.synchronize()
    assert_workspace_zero()
    got = {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in out.items()}
    assert_parity(got, oracle_case(c), name)
    q, s = O.mxfp8_quantize(bits)
    assert np.array_equal(got["act_scale"], s), "E8M0 scales differ"
    bad = np.argwhere(got["act_q"] != q)
    assert bad.size == 0, f"E4M3 codes differ at {bad[:5].tolist()}"


def test_route_quant_rejects_bad_hidden():
    c = W.tiny_global(8)
    with pytest.raises(M.MoeRouteError):
        M.route_quant_local(to_dev(c.logits), to_dev(c.bias),
                            torch.zeros((8, 100), dtype=torch.int16, device="cuda"))
