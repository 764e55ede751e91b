"""GPU parity of prepare_indexer_q_mxfp4 (RoPE tail, Hadamard rotation, MXFP4 encode,
weight fold) against the CPU oracle on the same seeded inputs.

Bar: bit-exact on the packed E2M1 codes, the e8m0 scale bytes and the folded fp32
weights.  The codes are integers decided by floating point; both sides take every
decision in the same precision (fp32 RoPE with separately rounded products, bf16
rounding, the fp32 radix-2 fast Hadamard transform with index bit 0 first, one fp32
multiply by the scale, exact exponent rule).
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


def _compare(inp, tokens=None):
    vals, scales, w_out = sad.prepare_indexer_q_mxfp4(inp.index_q, inp.positions, inp.cos_sin, inp.weights,
                                                      inp.softmax_scale, inp.head_scale)
    torch.cuda.synchronize()
    T = inp.index_q.shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    ov, os_, ow = O.prepare_indexer_q_mxfp4(_bits(inp.index_q)[tok], inp.positions.cpu().numpy()[tok],
                                            inp.cos_sin.cpu().numpy(), inp.weights.cpu().numpy()[tok],
                                            inp.softmax_scale, inp.head_scale)
    gv, gs, gw = vals.cpu().numpy()[tok], scales.cpu().numpy()[tok], w_out.cpu().numpy()[tok]
    bad_v = np.argwhere(gv != ov)
    assert bad_v.size == 0, f"{len(bad_v)} value bytes differ, first {bad_v[:4].tolist()}"
    assert np.array_equal(gs, os_), "scale bytes differ"
    assert np.array_equal(gw.view(np.uint32), ow.view(np.uint32)), "folded weights differ"
    return vals, scales, w_out


@pytest.mark.parametrize("T,H,D,R,P", [(1, 4, 64, 32, 300), (7, 4, 64, 32, 300), (37, 64, 128, 64, 4096),
                                       (3, 1, 128, 64, 10), (5, 3, 128, 8, 64), (2, 64, 64, 56, 16)])
def test_small_shapes_all_rows(T, H, D, R, P):
    log(f"[qprep] T={T} H={H} D={D} R={R} P={P}")
    pos = torch.randint(0, P, (T,), generator=torch.Generator().manual_seed(T))
    pos[0] = P - 1
    if T > 2:
        pos[1] = -1  # outside the table: failed closed
        pos[2] = P
    inp = WL.make_indexer_q_inputs(T, H, D, R, P, seed=100 + T, device="cuda", positions=pos)
    vals, scales, w = _compare(inp)
    if T > 2:
        assert not vals[1:3].any() and not scales[1:3].any() and not w[1:3].any()


def test_grid_ties_and_extreme_scales():
    # D = 64: the rotation scale is 1/8, so rows a*e0 + b*e1 rotate to exactly (a +- b)/8
    # and land on E2M1 midpoints; other rows are scaled by 2^+-40 and 2^-120.
    T, H, D, R, P = 4, 6, 64, 32, 8
    inp = WL.make_indexer_q_inputs(T, H, D, R, P, seed=9, device="cuda", positions=[0, 1, 2, 3])
    q = torch.zeros(T, H, D)
    for h, (a, b) in enumerate([(44, 4), (26, 2), (10, 2), (6, 2), (3, 1), (0, 0)]):
        q[0, h, 0], q[0, h, 1] = a, b
    q[1] = torch.randn(H, D) * 2.0 ** 40
    q[2] = torch.randn(H, D) * 2.0 ** -40
    q[3] = torch.randn(H, D) * 2.0 ** -120
    inp.index_q = q.bfloat16().cuda()
    vals, scales, _ = _compare(inp)
    v0 = vals[0].cpu().numpy()
    codes = np.stack([v0 & 0xF, v0 >> 4], -1).reshape(H, D)
    assert codes[0, 0] == 7 and codes[0, 1] == 6  # 6 and the 4/6 midpoint 5 -> 4 (code 6)
    assert not codes[5].any() and int(scales[0, 5, 0]) == 0  # zero row


def test_decode_batch_128_tokens_64_heads_at_64k():
    # The decode shape of the 128-request, 64K-context step: 128 tokens at position
    # 65535, 64 indexer heads of 128, rope 64; every token computed on the GPU, a
    # sample checked against the oracle.
    T, H, D, R, P = 128, 64, 128, 64, 65536
    inp = WL.make_indexer_q_inputs(T, H, D, R, P, seed=21, device="cuda", positions=[P - 1] * T)
    _compare(inp, tokens=[0, 1, 63, 64, 126, 127])


def test_prefill_16448_tokens_sampled():
    T, H, D, R, P = 16448, 64, 128, 64, 32768
    inp = WL.make_indexer_q_inputs(T, H, D, R, P, seed=22, device="cuda")
    rng = np.random.default_rng(3)
    tokens = sorted(set([0, 1, T - 1] + rng.integers(0, T, 13).tolist()))
    vals, scales, w = _compare(inp, tokens=tokens)
    again = sad.prepare_indexer_q_mxfp4(inp.index_q, inp.positions, inp.cos_sin, inp.weights,
                                        inp.softmax_scale, inp.head_scale)
    assert torch.equal(again[0], vals) and torch.equal(again[1], scales) and torch.equal(again[2], w)
