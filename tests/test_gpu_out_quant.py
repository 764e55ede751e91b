"""GPU parity of inv_rope_fp8_quant (inverse RoPE of each head's tail, heads grouped,
power-of-two FP8 blocks of 128) against the CPU oracle on the same seeded inputs.

Bar: bit-exact on the e4m3fn codes and on the fp32 scales.  The codes are integers
decided by floating point; both sides rotate with the same separately rounded fp32
operations and take the same exact exponent rule.
"""

import numpy as np
import pytest
import torch

import sparse_attention_decode_build_amd as sad
from oracle import sad_oracle as O
from sparse_attention_decode_build_amd import workloads as WL

from gpu_helpers import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sad.load()
    yield


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _compare(o, pos, cs, G, R, tokens=None):
    codes, scales = sad.inv_rope_fp8_quant(o, pos, cs, G)
    torch.cuda.synchronize()
    T = o.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    oc, osc = O.inv_rope_fp8_quant(_bits(o)[tok], pos.cpu().numpy()[tok], cs.cpu().numpy(), G, R)
    gc, gs = codes.cpu().numpy()[:, tok], scales.cpu().numpy()[:, tok]
    bad = np.argwhere(gc != oc)
    assert bad.size == 0, f"{len(bad)} codes differ, first (g, t, d) {bad[:4].tolist()}"
    assert np.array_equal(gs.view(np.uint32), osc.view(np.uint32)), "scales differ"
    return codes, scales


def _inputs(T, H, Dh, R, P, seed, positions=None, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    o = (torch.randn(T, H, Dh, generator=g) * scale).bfloat16()
    if positions is None:
        positions = torch.randint(0, P, (T,), generator=g)
    pos = torch.as_tensor(positions, dtype=torch.int32)
    return o.cuda(), pos.cuda(), WL.rope_table(P, R).cuda()


@pytest.mark.parametrize("T,H,Dh,R,G,P", [(3, 8, 576, 64, 2, 40), (5, 16, 512, 64, 4, 100),
                                          (2, 4, 160, 32, 1, 50), (1, 128, 576, 64, 16, 65536),
                                          (4, 2, 64, 64, 1, 8)])
def test_small_shapes_all_rows(T, H, Dh, R, G, P):
    log(f"[outq] T={T} H={H} Dh={Dh} R={R} G={G} P={P}")
    pos = torch.randint(0, P, (T,), generator=torch.Generator().manual_seed(T))
    pos[0] = P - 1
    if T > 2:
        pos[1] = -1
        pos[2] = P
    o, pos, cs = _inputs(T, H, Dh, R, P, seed=200 + T, positions=pos, scale=0.03)
    codes, scales = _compare(o, pos, cs, G, R)
    if T > 2:
        assert not codes[:, 1:3].any() and not scales[:, 1:3].any()


def test_e4m3_midpoints_subnormals_and_extreme_blocks():
    # Position 0 leaves the values unrotated.  Block 0 of each row holds 448 * 2^-8
    # with every e4m3 midpoint below it (ties to even), block 1 values in the e4m3
    # subnormal range of its scale, block 2 is zero, block 3 holds huge values.
    T, H, Dh, R, G, P = 1, 2, 256, 64, 1, 4
    vals = torch.from_numpy(O.E4M3_VALUES[:127].copy()).float()
    mids = ((vals[:-1] + vals[1:]) / 2)
    o = torch.zeros(T, H, Dh)
    row = o.view(-1)
    row[0] = 448.0 * 2.0 ** -8
    row[1:127] = mids[:126][: 126] * 2.0 ** -8 * torch.where(torch.arange(126) % 2 == 0, 1.0, -1.0)
    row[128] = 448.0
    row[129:160] = torch.arange(1, 32).float() * 2.0 ** -10
    row[384:400] = torch.linspace(-3e37, 3e37, 16)
    o = o.bfloat16()
    assert torch.equal(o.float().view(-1)[1:127], row[1:127])  # midpoints are exact in bf16
    _compare(o.cuda(), torch.tensor([0], dtype=torch.int32).cuda(), WL.rope_table(P, R).cuda(), G, R)


def test_decode_batch_128_tokens_at_64k_sampled():
    T, H, Dh, R, G, P = 128, 128, 576, 64, 16, 65536
    o, pos, cs = _inputs(T, H, Dh, R, P, seed=41, positions=[P - 1] * T, scale=0.03)
    _compare(o, pos, cs, G, R, tokens=[0, 77, 127])


def test_prefill_16448_tokens_sampled():
    T, H, Dh, R, G, P = 16448, 128, 576, 64, 16, 32768
    o, pos, cs = _inputs(T, H, Dh, R, P, seed=42, scale=0.03)
    codes, scales = _compare(o, pos, cs, G, R, tokens=[0, 5000, T - 1])
    again = sad.inv_rope_fp8_quant(o, pos, cs, G)
    assert torch.equal(again[0], codes) and torch.equal(again[1], scales)
