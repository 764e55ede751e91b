"""Pins of the CPU oracle against facts outside itself (CPU only).

Each test checks one oracle step against a library routine, a value printed
on the pages (fixtures under tests/golden/), a closed form, an invariant or
brute force, chosen so a plausible slip (wrong nibble order, wrong scale
block, dropped ReLU, off-by-one window, transposed operand) fails one of them.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import sad_oracle as O
from sparse_attention_decode_build_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# --------------------------------------------------------------------------- codecs


def test_e4m3_matches_torch_cast_all_bytes():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    mine = O.E4M3_VALUES
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0xFE] == -448.0  # largest finite
    assert mine[0x01] == 2.0 ** -9  # smallest subnormal


def test_e2m1_matches_printed_table():
    for nib, val in _golden("e2m1_table.txt"):
        v = float(val)
        got = O.e2m1_value(int(nib))
        assert got == v and math.copysign(1, got) == math.copysign(1, v) or (v == 0 and got == 0)


def test_fp8_max_and_blocks_match_pages():
    consts = {k: float(v) for k, v in _golden("format_constants.txt")}
    assert consts["fp8_max"] == float(torch.finfo(torch.float8_e4m3fn).max)
    assert consts["fp8_max"] == max(O.E4M3_VALUES[~np.isnan(O.E4M3_VALUES)])
    assert WL.FP8_BLOCK == consts["fp8_block"] and WL.MX_BLOCK == consts["mxfp4_block"]


def test_e8m0_is_power_of_two():
    for b in range(255):
        assert O.e8m0_value(b) == math.ldexp(1.0, b - 127)


def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1_000_000).astype(np.float32) * np.float32(3.0)
    # exact ties (low 16 bits 0x8000) with both parities, plus specials
    u = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    ties = ties[np.isfinite(ties)]
    specials = np.array([0.0, -0.0, 1e-40, -1e-40, 3.0e38, np.inf, -np.inf], np.float32)
    x = np.concatenate([x, ties, specials])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.float32_to_bf16_bits(x), ref)
    back = O.bf16_bits_to_float(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_mxfp4_nibble_order_and_block_scale():
    # low nibble is the even element, high nibble the odd one; one scale per 32
    packed = np.zeros((1, 32), np.uint8)
    packed[0, 0] = 0x2F  # element0 = nibble 0xF = -6, element1 = nibble 0x2 = 1.0
    packed[0, 16] = 0x71  # element32 = 0.5, element33 = 6
    exps = np.array([[127 + 1, 127 - 2]], np.uint8)  # block0 x2, block1 x1/4
    v = O.mxfp4_decode(packed, exps)
    assert v[0, 0] == -12.0 and v[0, 1] == 2.0
    assert v[0, 32] == 0.5 * 0.25 and v[0, 33] == 6.0 * 0.25
    assert np.count_nonzero(v) == 4


def test_mxfp4_encoder_roundtrip_within_half_step():
    # write side (workload encoder) and read side (oracle) were written apart;
    # the decoded value must be the nearest grid point at the block's scale.
    x = torch.randn(512, 64, generator=torch.Generator().manual_seed(1))
    packed, exps = WL.encode_mxfp4(x)
    v = O.mxfp4_decode(packed.numpy(), exps.numpy())
    xs = x.double().numpy()
    scale = np.repeat(np.ldexp(1.0, exps.numpy().astype(np.int64) - 127), 32, axis=1)
    grid = np.array(sorted(set(abs(g) for g in O.E2M1_VALUES)))
    y = np.abs(xs) / scale
    nearest = np.min(np.abs(y[..., None] - grid), axis=-1)
    assert np.all(np.abs(np.abs(v) / scale - y) <= nearest + 1e-12)
    assert np.all(np.abs(xs) / scale <= 6.0 + 1e-9)


# --------------------------------------------------------------------------- dequant


def _one_page_cache(rows_bf16, B, Dn, Dr):
    cfg = WL.Config(name="t", seed=0, window=1, ratio=1, topk=1, heads=1, d_nope=Dn, d_rope=Dr,
                    idx_heads=1, idx_dim=64, block=B, idx_block=B)
    page = WL._kv_page_bytes(cfg, rows_bf16)
    return {7: page[0].numpy()}, cfg


def test_dequant_roundtrip_bound_and_idempotence():
    B, Dn, Dr = 16, 128, 32
    g = torch.Generator().manual_seed(3)
    x = torch.randn(B, Dn + Dr, generator=g)
    x[3, :64] *= 1e-3  # small block: exercises subnormal codes
    x[5, 64:128] = 0.0  # all-zero block: amax clamped
    x = x.to(torch.bfloat16)
    pages, _ = _one_page_cache(x, B, Dn, Dr)
    slots = np.arange(7 * B, 8 * B)
    got = O.dequant_rows(pages, slots, B, Dn, Dr)
    xh = O.bf16_bits_to_float(got)
    xr = x.double().numpy()
    scale = np.repeat(
        np.maximum(np.abs(xr[:, :Dn]).reshape(B, -1, 64).max(-1), 1e-4) / 448.0, 64, axis=1)
    err = np.abs(xh[:, :Dn] - xr[:, :Dn])
    assert np.all(err <= (2 ** -4 + 2 ** -8) * np.abs(xr[:, :Dn]) + 2 ** -9 * scale * 1.0001)
    assert np.array_equal(got[:, Dn:], x[:, Dn:].view(torch.int16).numpy().view(np.uint16))
    # idempotence: re-encoding the dequantized value with the stored scale gives the same byte
    page = pages[7]
    row_b = Dn + 2 * Dr
    sc = page[B * row_b:].view(np.float32).reshape(B, Dn // 64)
    codes = np.stack([page[o * row_b: o * row_b + Dn] for o in range(B)])
    re = torch.from_numpy(
        (xh[:, :Dn] / np.repeat(sc.astype(np.float64), 64, axis=1)).astype(np.float32)
    ).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(re, codes)


def test_dequant_reads_the_addressed_row_and_scale_block():
    # closed form on a hand-built page: row o, block b holds byte 0x38 (=1.0) and
    # scale (o + 1) * 2^b, so every dequantized element is exactly (o + 1) * 2^b.
    B, Dn, Dr = 16, 128, 32
    row_b = Dn + 2 * Dr
    page = np.zeros(B * (row_b + 4 * (Dn // 64)), np.uint8)
    for o in range(B):
        page[o * row_b: o * row_b + Dn] = 0x38
        sc = np.array([(o + 1) * 2.0 ** b for b in range(Dn // 64)], np.float32)
        page[B * row_b + o * 8: B * row_b + o * 8 + 8] = sc.view(np.uint8)
    got = O.bf16_bits_to_float(O.dequant_rows({2: page}, [2 * B + 5, -1, 2 * B], B, Dn, Dr))
    assert np.all(got[0, :64] == 6.0) and np.all(got[0, 64:Dn] == 12.0)
    assert np.all(got[1] == 0.0)
    assert np.all(got[2, :64] == 1.0) and np.all(got[2, 64:Dn] == 2.0)


def test_dequant_native_ue8m0_record():
    # The pages' native record: 448 e4m3 + 64 bf16 per row (576 bytes), then per row 8
    # scale bytes (7 ue8m0 + 1 pad).  Row o, block b: byte 0x38 (= 1.0) with scale byte
    # 120 + b + o % 3, so element d is exactly 2^(d // 64 + o % 3 - 7); the pad byte is
    # 0xFF and must be ignored; the rope part is copied.
    B, Dn, Dr = 16, 448, 64
    row_b = Dn + 2 * Dr
    assert O.kv_scale_bytes(Dn, "ue8m0") == 8 and row_b == 576
    page = np.zeros(B * (row_b + 8), np.uint8)
    rope = (np.arange(Dr, dtype=np.float32) - 20.5).astype(np.float32)
    for o in range(B):
        page[o * row_b: o * row_b + Dn] = 0x38
        page[o * row_b + Dn: (o + 1) * row_b] = O.float32_to_bf16_bits(rope * (o + 1)).view(np.uint8)
        page[B * row_b + 8 * o: B * row_b + 8 * o + 7] = 120 + np.arange(7) + o % 3
        page[B * row_b + 8 * o + 7] = 0xFF
    got = O.bf16_bits_to_float(O.dequant_rows({1: page}, [B + 4, -1, B + 8], B, Dn, Dr, "ue8m0"))
    for r, o in ((0, 4), (2, 8)):
        want = np.exp2(np.arange(Dn) // 64 + o % 3 - 7.0)
        assert np.array_equal(got[r, :Dn], want)
        assert np.array_equal(got[r, Dn:], O.bf16_bits_to_float(O.float32_to_bf16_bits(rope * (o + 1))))
    assert not got[1].any()


# --------------------------------------------------------------------------- geometry / indices


def test_positions_closed_form():
    qsl = [0, 1, 4, 4, 6]
    seq = [10, 3, 7, 2]
    t2r = [0, 1, 1, 1, 3, 3]
    pos = O.token_positions(qsl, seq, t2r)
    assert pos.tolist() == [9, 0, 1, 2, 0, 1]
    assert O.compressed_len(np.array([0, 2, 3, 4, 7, 127]), 4).tolist() == [0, 0, 1, 1, 2, 32]
    with pytest.raises(ValueError):
        O.token_positions([0, 1], [5], [0, 0])


def _random_batch(rng, R=6, B=4, W=5, ratio=4, topk=6, P=8, pages=200):
    q_lens = rng.integers(0, 5, R)
    seq = np.array([int(rng.integers(ql, ql + 40)) if ql else int(rng.integers(1, 40)) for ql in q_lens])
    qsl = np.concatenate([[0], np.cumsum(q_lens)])
    t2r = np.repeat(np.arange(R), q_lens)
    replay = rng.integers(0, 20, R)
    cols = (seq.max() + B - 1) // B + 1
    perm = rng.permutation(pages)
    swa_bt = perm[: R * cols].reshape(R, cols).astype(np.int32)
    comp_bt = perm[R * cols: 2 * R * cols].reshape(R, cols).astype(np.int32)
    swa_bt[rng.random(swa_bt.shape) < 0.15] = -1  # unbacked pages
    comp_bt[rng.random(comp_bt.shape) < 0.15] = -1
    comp_bt[0, 0] = pages + 5  # past the pool: invalid
    T = int(q_lens.sum())
    topk_local = rng.integers(-2, 14, (T, topk + 2)).astype(np.int32)
    return dict(qsl=qsl, seq=seq, t2r=t2r, replay=replay, swa_bt=swa_bt, comp_bt=comp_bt,
                topk_local=topk_local, B=B, W=W, ratio=ratio, topk=topk, P=P, pages=pages)


@pytest.mark.parametrize("seed", range(8))
def test_sparse_indices_match_brute_force(seed):
    rng = np.random.default_rng(seed)
    b = _random_batch(rng)
    dense = seed % 2 == 1
    tk = None if dense else b["topk_local"]
    si, lens = O.build_sparse_indices(
        b["qsl"], b["seq"], b["t2r"], b["replay"], b["swa_bt"], b["B"], b["pages"],
        b["comp_bt"], b["B"], b["pages"], tk, b["topk"], b["W"], b["ratio"], b["P"])
    # independent walk: enumerate every position of the request, keep the window
    for t, r in enumerate(b["t2r"]):
        qlen = b["qsl"][r + 1] - b["qsl"][r]
        p = b["seq"][r] - qlen + (t - b["qsl"][r])
        keep = [x for x in range(0, p + 1) if x > p - b["W"] and x >= b["replay"][r]]
        exp_swa = []
        for x in keep:
            page = b["swa_bt"][r][x // b["B"]] if x // b["B"] < b["swa_bt"].shape[1] else -1
            exp_swa.append(int(page) * b["B"] + x % b["B"] if 0 <= page < b["pages"] else -1)
        exp_swa += [-1] * (b["W"] - len(exp_swa))
        assert si[t, : b["W"]].tolist() == exp_swa
        nc = (p + 1) // b["ratio"]
        cand = list(range(min(nc, b["P"]))) if dense else b["topk_local"][t, : b["topk"]].tolist()
        exp_c = []
        for l in cand:
            if 0 <= l < nc:
                page = b["comp_bt"][r][l // b["B"]]
                if 0 <= page < b["pages"]:
                    exp_c.append(int(page) * b["B"] + l % b["B"])
        assert lens[t] == len(exp_c)
        assert si[t, b["W"]:].tolist() == exp_c + [-1] * (b["P"] - len(exp_c))


def test_window_is_last_w_positions_clipped_by_replay():
    B, W = 4, 6
    bt = np.arange(10, dtype=np.int32)[None, :]  # identity table: slot == position
    for p in range(0, 30):
        for replay in (0, 3, p, p + 1):
            si, lens = O.build_sparse_indices([0, 1], [p + 1], [0], [replay], bt, B, 100, bt, B, 100,
                                              None, 0, W, 4, 64)
            want = list(range(max(p - W + 1, replay, 0), p + 1))
            assert si[0, :W].tolist() == want + [-1] * (W - len(want))
            assert lens[0] == min((p + 1) // 4, 64)


# --------------------------------------------------------------------------- indexer / top-k


def _mx_query(rng, H, D):
    x = torch.from_numpy(rng.standard_normal((H, D)).astype(np.float32))
    v, e = WL.encode_mxfp4(x)
    return v.numpy(), e.numpy()


# E2M1 magnitudes as the [ops] page prints them (codes 0..7; bit 3 is the sign)
_E2M1_PRINTED = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _mx_page(B, dim, code_of, exp_of):
    """A hand-built indexer key page: B rows of dim/2 packed bytes (element 2k in the low
    nibble of byte k), then B rows of dim/32 exponent bytes."""
    vb, sb = dim // 2, dim // 32
    page = np.zeros(B * (vb + sb), np.uint8)
    for o in range(B):
        for k in range(vb):
            page[o * vb + k] = code_of(o, 2 * k) | (code_of(o, 2 * k + 1) << 4)
        for b in range(sb):
            page[B * vb + o * sb + b] = exp_of(o, b)
    return page


def test_read_index_keys_hand_built_page_and_unbacked_rows():
    """[ops] read_deepseek_v4_indexer_mxfp4_cache: the value region (B x dim/2 bytes, low
    nibble = even element) comes before the exponent region (B x dim/32 e8m0 bytes).  Row o,
    element d of the page holds code (d + 3o) % 8 with the sign bit where (d + o) % 5 == 0,
    and block b of row o the exponent byte 120 + o + 3b, so the key is
    +-E2M1[(d + 3o) % 8] * 2^(o + 3b - 7).  The table names an unbacked page (-1), a page
    past the pool and (by its length) no page for the last rows: those rows are invalid
    and read as zero."""
    B, dim = 16, 64
    code = lambda o, d: ((d + 3 * o) % 8) | (0x8 if (d + o) % 5 == 0 else 0)  # noqa: E731
    expo = lambda o, b: 120 + o + 3 * b  # noqa: E731
    page = _mx_page(B, dim, code, expo)
    num_pages = 10
    bt_row = np.array([-1, 5, 99, 5], np.int32)  # logical pages 0..3; 99 is past the pool
    rows = 4 * B + 6  # 6 rows past the table
    keys, valid = O.read_index_keys({5: page}, bt_row, rows, B, dim, num_pages)
    want_valid = np.zeros(rows, bool)
    want_valid[B: 2 * B] = True
    want_valid[3 * B: 4 * B] = True
    assert np.array_equal(valid, want_valid)
    for lp in (1, 3):
        for o in range(B):
            want = np.array([(-1.0 if (d + o) % 5 == 0 else 1.0) * _E2M1_PRINTED[(d + 3 * o) % 8]
                             * 2.0 ** (o + 3 * (d // 32) - 7) for d in range(dim)])
            assert np.array_equal(keys[lp * B + o], want), (lp, o)
    assert not keys[~valid].any()
    # a row past n_c is never read: fewer rows than the table covers
    k2, v2 = O.read_index_keys({5: page}, bt_row, B + 3, B, dim, num_pages)
    assert k2.shape == (B + 3, dim) and np.array_equal(v2, want_valid[: B + 3])
    assert np.array_equal(k2[B:], keys[B: B + 3])


def test_indexer_topk_never_selects_unbacked_rows():
    """Rows whose key page is unbacked score nothing: top-k draws only from backed rows and
    pads with -1 when fewer than k are backed ([backend] safe_page_ids, fail closed)."""
    B, dim, H = 16, 64, 2
    rng = np.random.default_rng(12)
    pages = {}
    for pid in (2, 7):
        keys = torch.from_numpy(rng.standard_normal((B, dim)).astype(np.float32))
        v, e = WL.encode_mxfp4(keys)
        pages[pid] = np.concatenate([v.numpy().reshape(-1), e.numpy().reshape(-1)])
    idx_bt = np.array([[2, -1, 7, 40]], np.int32)  # 40: past a pool of 10 pages
    qv, qe = _mx_query(rng, H, dim)
    w = np.abs(rng.standard_normal(H))
    seq = 4 * B * 4  # n_c = 64 rows: logical pages 0..3
    out, sc = O.indexer_topk(np.array([0, 1]), np.array([seq]), np.array([0]), qv[None], qe[None], w[None],
                             pages, idx_bt, B, dim, 10, 4, 40, return_scores=True)
    scores, valid = sc[0]
    assert np.array_equal(np.nonzero(valid)[0], np.r_[0:B, 2 * B:3 * B])
    got = out[0]
    assert np.all(got[:2 * B] >= 0) and np.all(got[2 * B:] == -1)  # 32 backed rows < k = 40
    assert set(got[:2 * B].tolist()) == set(range(B)) | set(range(2 * B, 3 * B))


def test_scores_one_hot_query_reads_single_key_element():
    rng = np.random.default_rng(5)
    D = 64
    keys = torch.from_numpy(rng.standard_normal((10, D)).astype(np.float32))
    kv, ke = WL.encode_mxfp4(keys)
    kd = O.mxfp4_decode(kv.numpy(), ke.numpy())
    for i in (0, 1, 31, 32, 63):
        q = np.zeros((1, D // 2), np.uint8)
        q[0, i // 2] = 0x2 << (4 * (i % 2))  # element i = 1.0
        qe = np.full((1, D // 32), 127, np.uint8)
        s = O.indexer_scores(q, qe, np.array([1.0]), kd)
        assert np.array_equal(s, np.maximum(kd[:, i], 0.0))


def test_scores_relu_per_head_and_invariants():
    rng = np.random.default_rng(6)
    H, D, n = 4, 64, 50
    qv, qe = _mx_query(rng, H, D)
    neg = qv ^ np.uint8(0x88)  # flip both sign bits: q -> -q
    keys = O.mxfp4_decode(*[a.numpy() for a in WL.encode_mxfp4(torch.randn(n, D))])
    w = rng.standard_normal(H)
    s_pos = O.indexer_scores(qv, qe, w, keys)
    s_neg = O.indexer_scores(neg, qe, w, keys)
    qd = O.mxfp4_decode(qv, qe)
    dots = qd @ keys.T
    # relu applied per head: s(q) + s(-q) = sum_h w_h |q_h . k|
    assert np.allclose(s_pos + s_neg, w @ np.abs(dots), rtol=1e-12, atol=1e-12)
    assert np.allclose(s_pos - s_neg, w @ dots, rtol=1e-12, atol=1e-12)
    # head permutation invariance, weight homogeneity
    perm = rng.permutation(H)
    assert np.allclose(O.indexer_scores(qv[perm], qe[perm], w[perm], keys), s_pos, rtol=1e-12)
    assert np.array_equal(O.indexer_scores(qv, qe, 2 * w, keys), 2 * s_pos)
    # every per-head dot product is exact in binary32 (any summation order)
    assert np.array_equal(dots.astype(np.float32).astype(np.float64), dots)


def test_topk_brute_force():
    rng = np.random.default_rng(7)
    for trial in range(200):
        n = int(rng.integers(0, 30))
        k = int(rng.integers(1, 12))
        scores = np.round(rng.standard_normal(n), 1)  # many ties
        valid = rng.random(n) < 0.8
        got = O.topk_select(scores, valid, k)
        cand = [i for i in range(n) if valid[i]]
        chosen = []
        for _ in range(min(k, len(cand))):
            best = max(cand, key=lambda i: (scores[i], -i))
            chosen.append(best)
            cand.remove(best)
        want = sorted(chosen) + [-1] * (k - len(chosen))
        assert got.tolist() == want


def test_topk_special_cases():
    s = np.array([3.0, 1.0, 2.0])
    assert O.topk_select(s, np.ones(3, bool), 5).tolist() == [0, 1, 2, -1, -1]
    assert O.topk_select(s, np.ones(3, bool), 1).tolist() == [0]
    assert O.topk_select(np.zeros(6), np.ones(6, bool), 3).tolist() == [0, 1, 2]
    assert O.topk_select(np.zeros(0), np.zeros(0, bool), 2).tolist() == [-1, -1]


# --------------------------------------------------------------------------- attention


def _bf16_bits(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_attend_matches_library_softmax():
    from scipy.special import logsumexp, softmax

    rng = np.random.default_rng(8)
    H, n, D = 5, 37, 24
    q = _bf16_bits(rng.standard_normal((H, D)))
    x = _bf16_bits(rng.standard_normal((n, D)))
    sink = rng.standard_normal(H)
    qf, xf = O.bf16_bits_to_float(q), O.bf16_bits_to_float(x)
    c = D ** -0.5
    o, lse = O.attend(q, x, c, sink)
    logits = np.concatenate([c * qf @ xf.T, sink[:, None]], axis=1)
    p = softmax(logits, axis=1)
    assert np.allclose(o, p[:, :n] @ xf, rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, logsumexp(logits, axis=1), rtol=1e-12)
    o2, _ = O.attend(q, x, c, np.full(H, -np.inf))
    o3, _ = O.attend(q, x, c, None)
    assert np.allclose(o2, o3, rtol=1e-14, atol=0)


def test_attend_degenerate_cases():
    rng = np.random.default_rng(9)
    q = _bf16_bits(rng.standard_normal((3, 16)))
    x0 = _bf16_bits(rng.standard_normal((1, 16)))
    o, _ = O.attend(q, x0, 0.25)
    assert np.array_equal(o, np.repeat(O.bf16_bits_to_float(x0), 3, axis=0))  # single key
    o, _ = O.attend(q, np.repeat(x0, 9, axis=0), 0.25)
    assert np.allclose(o, np.repeat(O.bf16_bits_to_float(x0), 3, axis=0), rtol=1e-14)  # identical keys
    o, lse = O.attend(q, np.zeros((0, 16), np.uint16), 0.25)
    assert np.all(o == 0) and np.all(lse == -np.inf)  # empty set


def test_sparse_equals_dense_when_everything_is_selected():
    """topk >= n_c and window >= seq_len: the sparse step equals dense attention
    over every compressed row and every position, computed by torch SDPA in
    float64 over rows reached by walking the block tables directly."""
    cfg = WL.with_overrides(WL.CONFIGS["tiny"], window=256, topk=64)
    wl = WL.make_workload(cfg, "cpu")
    v = WL.host_view(wl)
    P = wl.padded_topk
    res = O.step(v, cfg, P, wl.kv_pool.shape[0], wl.idx_pool.shape[0], wl.softmax_scale)
    # the whole history was selected
    assert res["lens"][0] == 64 and np.all(res["sparse_indices"][0] >= 0)
    rows_swa = [O.logical_to_slot(v.swa_bt[0], p, cfg.block, 10**9) for p in range(256)]
    rows_cmp = [O.logical_to_slot(v.comp_bt[0], l, cfg.block, 10**9) for l in range(64)]
    rows = O.dequant_rows(v.kv_pages, rows_swa + rows_cmp, cfg.block, cfg.d_nope, cfg.d_rope)
    x = torch.from_numpy(O.bf16_bits_to_float(rows))[None, None]  # [1,1,n,D]
    q = torch.from_numpy(O.bf16_bits_to_float(v.q[0]))[None, :, None, :]  # [1,H,1,D]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, x.expand(1, cfg.heads, -1, -1), x.expand(1, cfg.heads, -1, -1), scale=wl.softmax_scale)
    assert np.allclose(res["out"][0], ref[0, :, 0].numpy(), rtol=1e-10, atol=1e-12)


def test_sparse_attention_ignores_padding_and_invalid_columns():
    cfg = WL.CONFIGS["tiny"]
    wl = WL.make_workload(cfg, "cpu")
    v = WL.host_view(wl)
    P = wl.padded_topk
    res = O.step(v, cfg, P, wl.kv_pool.shape[0], wl.idx_pool.shape[0], wl.softmax_scale)
    si = res["sparse_indices"].copy()
    lens = res["lens"]
    W = cfg.window
    # garbage past lens and -1 anywhere must not change the result
    si2 = si.copy()
    si2[0, W + lens[0]:] = si[0, W]  # a valid slot, but past lens
    o2, _ = O.sparse_mla_decode(v.q, v.kv_pages, v.kv_pages, si2, lens, W, cfg.block, cfg.block,
                                cfg.d_nope, cfg.d_rope, wl.softmax_scale)
    assert np.array_equal(o2, res["out"])


def _const_kv_page(B, Dn, Dr, byte, scale, rope_val):
    """A KV page whose every row is byte `byte` (e4m3) with fp32 scale `scale` per block and
    rope elements `rope_val` (bf16)."""
    row_b = Dn + 2 * Dr
    page = np.zeros(B * (row_b + 4 * (Dn // 64)), np.uint8)
    rope = O.float32_to_bf16_bits(np.full(Dr, rope_val, np.float32)).view(np.uint8)
    for o in range(B):
        page[o * row_b: o * row_b + Dn] = byte
        page[o * row_b + Dn: (o + 1) * row_b] = rope
        page[B * row_b + o * 4 * (Dn // 64): B * row_b + (o + 1) * 4 * (Dn // 64)] = \
            np.full(Dn // 64, scale, np.float32).view(np.uint8)
    return page


def test_window_and_compressed_columns_read_their_own_caches():
    """[backend] forward_deepseek_v4_decode passes the window cache as k_cache and the
    compressed cache as extra_k_cache, each with its own page size.  Window columns must
    read the window cache and compressed columns the compressed one: page 3 exists in both
    with different bytes (x = 1 / rope 0.5 in the window cache, x = -2 / rope -0.25 in the
    compressed one)."""
    Dn, Dr = 128, 32
    for Bs, Bc in ((16, 16), (64, 16), (16, 64)):
        swa = {3: _const_kv_page(Bs, Dn, Dr, 0x38, 1.0, 0.5)}    # e4m3 0x38 = 1.0
        comp = {3: _const_kv_page(Bc, Dn, Dr, 0xB8, 2.0, -0.25)}  # e4m3 0xB8 = -1.0
        W, P = 4, 4
        si = np.array([[3 * Bs + 1, -1, 3 * Bs + Bs - 1, 3 * Bs,
                        3 * Bc + 2, 3 * Bc + 5, 3 * Bc, 3 * Bc + 7]], np.int32)
        lens = np.array([2], np.int32)  # compressed columns past lens are not attended
        got = O.bf16_bits_to_float(O.gather_dequant(swa, comp, si, lens, W, Bs, Bc, Dn, Dr))[0]
        for c in (0, 2, 3):
            assert np.all(got[c, :Dn] == 1.0) and np.all(got[c, Dn:] == 0.5), (Bs, Bc, c)
        for c in (4, 5):
            assert np.all(got[c, :Dn] == -2.0) and np.all(got[c, Dn:] == -0.25), (Bs, Bc, c)
        for c in (1, 6, 7):
            assert not got[c].any()
        # attention: 3 window rows u and 2 compressed rows v, so
        # o = (3 e^{l_u} u + 2 e^{l_v} v) / (3 e^{l_u} + 2 e^{l_v})
        rng = np.random.default_rng(Bs + Bc)
        H = 4
        q = _bf16_bits(rng.standard_normal((1, H, Dn + Dr)))
        c_s = 0.05
        o, lse = O.sparse_mla_decode(q, swa, comp, si, lens, W, Bs, Bc, Dn, Dr, c_s)
        u = np.r_[np.full(Dn, 1.0), np.full(Dr, 0.5)]
        v = np.r_[np.full(Dn, -2.0), np.full(Dr, -0.25)]
        qf = O.bf16_bits_to_float(q[0])
        lu, lv = c_s * (qf @ u), c_s * (qf @ v)
        m = np.maximum(lu, lv)
        wu, wv = 3 * np.exp(lu - m), 2 * np.exp(lv - m)
        want = (wu[:, None] * u + wv[:, None] * v) / (wu + wv)[:, None]
        assert np.allclose(o[0], want, rtol=1e-13, atol=1e-13)
        assert np.allclose(lse[0], m + np.log(wu + wv), rtol=1e-13)


def test_attention_spread_bounds_a_rounding_of_every_weight():
    """attention_spread(h, d) = sum_j p_j |x_j[d] - o[h, d]|: zero for one row, the closed
    form p(1-p)|x_0 - x_1| * 2 for two rows, and rounding every normalized weight to bf16
    (then renormalizing) moves the output by at most 2^-8 of it (brute force)."""
    rng = np.random.default_rng(21)
    H, D, n = 3, 16, 40
    q = _bf16_bits(rng.standard_normal((H, D)) * 3)
    x = _bf16_bits(rng.standard_normal((n, D)))
    c = 0.5
    heads = np.repeat(np.arange(H), D)
    dims = np.tile(np.arange(D), H)
    assert not O.attention_spread(q, x[:1], c, None, heads, dims).any()
    two = O.attention_spread(q, x[:2], c, None, heads, dims).reshape(H, D)
    xf = O.bf16_bits_to_float(x[:2])
    qf = O.bf16_bits_to_float(q)
    l = c * (qf @ xf.T)
    p0 = 1.0 / (1.0 + np.exp(l[:, 1] - l[:, 0]))
    want = 2 * (p0 * (1 - p0))[:, None] * np.abs(xf[0] - xf[1])[None, :]
    assert np.allclose(two, want, rtol=1e-12, atol=1e-15)
    sp = O.attention_spread(q, x, c, None, heads, dims).reshape(H, D)
    o, _ = O.attend(q, x, c)
    xf = O.bf16_bits_to_float(x)
    lg = c * (O.bf16_bits_to_float(q) @ xf.T)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    pb = O.bf16_bits_to_float(O.float32_to_bf16_bits(p.astype(np.float32)))
    ob = (pb @ xf) / pb.sum(axis=1, keepdims=True)
    assert np.all(np.abs(ob - o) <= 2.0 ** -8 * sp + 1e-15)


# --------------------------------------------------------------------------- indexer query preparation


def test_mxfp4_encode_hand_worked_cases():
    for line in _golden("mxfp4_encode_cases.txt"):
        text = " ".join(line)
        sbyte, vals, codes = (part.strip() for part in text.split("|"))
        vals = [float(v) for v in vals.split()]
        codes = [int(c, 16) for c in codes.split()]
        x = np.zeros(32)
        x[: len(vals)] = vals
        packed, exps = O.mxfp4_encode(x[None, :])
        assert int(exps[0, 0]) == int(sbyte), text
        got = np.empty(32, dtype=np.int64)
        got[0::2] = packed[0] & 0xF
        got[1::2] = packed[0] >> 4
        assert list(got[: len(codes)]) == codes, text
        assert not got[len(codes):].any(), text


def test_mxfp4_encode_matches_threshold_encoder_and_error_bound():
    # The harness's write-side encoder is a separate implementation (rounding by
    # threshold counting, exponent from a float log2); on nonzero bf16 blocks the
    # two must give the same bytes.  The decode of the encoding is within half a
    # grid step: 2^e for |x| / 2^e in [4, 6], 2^(e-2) below 2.
    g = torch.Generator().manual_seed(7)
    x = (torch.randn(64, 128, generator=g) * torch.exp2(torch.randint(-8, 8, (64, 1), generator=g).float()))
    x = x.bfloat16().float()
    mine_v, mine_s = O.mxfp4_encode(x.numpy().astype(np.float64))
    ref_v, ref_s = WL.encode_mxfp4(x)
    assert np.array_equal(mine_v, ref_v.numpy()) and np.array_equal(mine_s, ref_s.numpy())
    dec = O.mxfp4_decode(mine_v, mine_s)
    scale = np.repeat(np.ldexp(1.0, mine_s.astype(np.int64) - 127), 32, axis=1)
    xv = x.numpy().astype(np.float64)
    err = np.abs(dec - xv)
    assert (err <= scale * 1.0).all()
    small = np.abs(xv) <= 2.0 * scale
    assert (err[small] <= 0.25 * scale[small]).all()
    amax = np.abs(xv).reshape(64, 4, 32).max(-1)
    e = mine_s.astype(np.float64) - 127
    assert (6.0 * np.exp2(e - 1) < amax).all() and (amax <= 6.0 * np.exp2(e)).all()


def test_hadamard_matrix_is_sylvester_and_rotation_is_an_involution():
    import scipy.linalg
    for n in (2, 8, 32, 64, 128):
        assert np.array_equal(O.hadamard_matrix(n), scipy.linalg.hadamard(n))
    # The float32 fast transform is H x: exactly on small integers (every partial sum
    # is exact in float32), and within its rounding bound (one float32 rounding per
    # stage) on random bf16 rows.
    g = np.random.default_rng(8)
    for n in (2, 16, 64, 128):
        xi = g.integers(-256, 257, (9, n)).astype(np.float32)
        assert np.array_equal(O.fwht_f32(xi).astype(np.float64), xi.astype(np.float64) @ scipy.linalg.hadamard(n).T)
    xb = torch.randn(50, 128, generator=torch.Generator().manual_seed(4)).bfloat16().float().numpy()
    ex = xb.astype(np.float64) @ scipy.linalg.hadamard(128).T
    bound = 7 * 2.0 ** -24 * np.abs(xb).sum(axis=1, keepdims=True) * 2
    assert (np.abs(O.fwht_f32(xb).astype(np.float64) - ex) <= bound).all()
    # H / sqrt(n) is orthonormal and symmetric, so rotating twice returns the row
    # (up to two bf16 roundings), and the norm is kept.
    g = torch.Generator().manual_seed(3)
    x = torch.randn(40, 128, generator=g).bfloat16()
    bits = x.view(torch.int16).numpy().view(np.uint16)
    once = O.hadamard_rotate(bits)
    twice = O.bf16_bits_to_float(O.hadamard_rotate(once))
    xf = x.float().numpy().astype(np.float64)
    assert np.allclose(twice, xf, rtol=0, atol=4 * 2.0 ** -8 * np.abs(xf).max())
    n0 = np.linalg.norm(xf, axis=1)
    n1 = np.linalg.norm(O.bf16_bits_to_float(once), axis=1)
    assert np.allclose(n0, n1, rtol=2.0 ** -7)
    # A basis vector e_j maps to column j of H, scaled: the sign pattern pins the order.
    for j in (0, 1, 5, 64, 127):
        e = np.zeros((1, 128), np.float32)
        e[0, j] = 1.0
        out = O.bf16_bits_to_float(O.hadamard_rotate(O.float32_to_bf16_bits(e)))[0]
        assert np.array_equal(np.sign(out), scipy.linalg.hadamard(128)[:, j])
        assert np.allclose(np.abs(out), 128 ** -0.5, rtol=2.0 ** -8)


def test_rope_tail_is_a_complex_rotation_of_interleaved_pairs():
    g = np.random.default_rng(11)
    D, R = 128, 64
    x = g.standard_normal((5, 3, D)).astype(np.float32)
    theta = g.uniform(-math.pi, math.pi, (5, R // 2))
    cos, sin = np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)
    out = O.rope_gptj_tail(x, cos, sin, R)
    assert np.array_equal(out[..., : D - R], x[..., : D - R])
    z = (x[..., D - R::2].astype(np.float64) + 1j * x[..., D - R + 1::2].astype(np.float64))
    w = z * (cos.astype(np.float64) + 1j * sin.astype(np.float64))[:, None, :]
    assert np.allclose(out[..., D - R::2], w.real, rtol=0, atol=4e-6 * np.abs(z).max())
    assert np.allclose(out[..., D - R + 1::2], w.imag, rtol=0, atol=4e-6 * np.abs(z).max())
    # angle 0 is the identity, a quarter turn maps (e, o) to (-o, e): both exact
    ident = O.rope_gptj_tail(x, np.ones((5, R // 2), np.float32), np.zeros((5, R // 2), np.float32), R)
    assert np.array_equal(ident, x)
    quarter = O.rope_gptj_tail(x, np.zeros((5, R // 2), np.float32), np.ones((5, R // 2), np.float32), R)
    assert np.array_equal(quarter[..., D - R::2], -x[..., D - R + 1::2])
    assert np.array_equal(quarter[..., D - R + 1::2], x[..., D - R::2])


def test_prepare_indexer_q_end_to_end_properties():
    # The prepared query decodes to the rotated query within the MXFP4 step, the
    # rotation keeps q . k (both sides rotated alike), the weights are folded, and
    # a position outside the table fails closed.
    g = np.random.default_rng(5)
    T, H, D, R, P = 4, 3, 128, 64, 50
    q = torch.from_numpy(g.standard_normal((T, H, D)).astype(np.float32)).bfloat16()
    qb = q.view(torch.int16).numpy().view(np.uint16)
    pos = np.array([0, 7, 49, 50])
    ang = np.outer(np.arange(P), 10000.0 ** (-np.arange(R // 2) * 2.0 / R))
    cs = np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)
    w = g.standard_normal((T, H)).astype(np.float32)
    vals, scales, w_out = O.prepare_indexer_q_mxfp4(qb, pos, cs, w, D ** -0.5, H ** -0.5)
    assert vals.shape == (T, H, D // 2) and scales.shape == (T, H, D // 32)
    assert not vals[3].any() and not scales[3].any() and not w_out[3].any()
    assert np.allclose(w_out[:3], w[:3].astype(np.float64) * D ** -0.5 * H ** -0.5, rtol=2.0 ** -22)
    dec = O.mxfp4_decode(vals.reshape(-1, D // 2), scales.reshape(-1, D // 32)).reshape(T, H, D)
    qf = q.float().numpy().astype(np.float64)
    for t in range(3):
        th = ang[pos[t]]
        z = (qf[t, :, D - R::2] + 1j * qf[t, :, D - R + 1::2]) * np.exp(1j * th)
        ideal = qf[t].copy()
        ideal[:, D - R::2], ideal[:, D - R + 1::2] = z.real, z.imag
        ideal = ideal @ O.hadamard_matrix(D) * D ** -0.5
        step = np.repeat(np.ldexp(1.0, scales[t].astype(np.int64) - 127), 32, axis=1)
        assert (np.abs(dec[t] - ideal) <= step + 2.0 ** -7 * np.abs(ideal)).all()
        k = g.standard_normal(D)
        krot = O.hadamard_matrix(D) @ k * D ** -0.5
        roped = qf[t].copy()
        roped[:, D - R::2], roped[:, D - R + 1::2] = z.real, z.imag
        assert np.allclose(dec[t] @ krot, roped @ k, rtol=0, atol=0.15 * np.linalg.norm(k) * np.abs(roped).max())


# --------------------------------------------------------------------------- output inverse RoPE + FP8


def test_fp8_pow2_scale_hand_worked_cases():
    for amax, e in _golden("fp8_pow2_scale_cases.txt"):
        b = np.zeros((1, 128))
        b[0, 5] = -float(amax)
        _, s = O.fp8_pow2_quant(b)
        assert s[0] == 2.0 ** int(e), (amax, e, s[0])


def test_e4m3_encode_matches_torch_cast():
    # torch's float8_e4m3fn cast rounds to nearest even; on values within +-448
    # (midpoints of every binade included) it must give the same bytes.
    vals = torch.from_numpy(O.E4M3_VALUES[:127].copy())
    mids = (vals[:-1] + vals[1:]) / 2
    g = torch.Generator().manual_seed(2)
    x = torch.cat([vals, -vals, mids, -mids, (torch.rand(20000, generator=g, dtype=torch.float64) - 0.5) * 896,
                   torch.randn(20000, generator=g, dtype=torch.float64) * 1e-2, torch.tensor([0.0, -0.0])])
    x = x.float()  # the quantizer's inputs are float32
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = O.e4m3_encode(x.numpy().astype(np.float64))
    assert np.array_equal(mine, ref)


def test_inv_rope_undoes_rope_and_is_a_conjugate_rotation():
    g = np.random.default_rng(12)
    D, R = 576, 64
    x = g.standard_normal((3, 4, D)).astype(np.float32)
    th = g.uniform(-math.pi, math.pi, (3, R // 2))
    c, s = np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
    inv = O.inv_rope_gptj_tail(x, c, s, R)
    assert np.array_equal(inv[..., : D - R], x[..., : D - R])
    z = x[..., D - R::2].astype(np.float64) + 1j * x[..., D - R + 1::2].astype(np.float64)
    w = z * (c.astype(np.float64) - 1j * s.astype(np.float64))[:, None, :]
    assert np.allclose(inv[..., D - R::2], w.real, atol=4e-6 * np.abs(z).max())
    assert np.allclose(inv[..., D - R + 1::2], w.imag, atol=4e-6 * np.abs(z).max())
    back = O.rope_gptj_tail(inv, c, s, R)
    assert np.allclose(back, x, rtol=0, atol=8e-6 * np.abs(x).max())
    quarter = O.inv_rope_gptj_tail(x, np.zeros_like(c), np.ones_like(s), R)
    assert np.array_equal(quarter[..., D - R::2], x[..., D - R + 1::2])
    assert np.array_equal(quarter[..., D - R + 1::2], -x[..., D - R::2])


def test_inv_rope_fp8_quant_layout_and_error_bound():
    # Group-major layout, blocks of 128 along the group's row (heads, then dims),
    # dequantized values within half an e4m3 step of the rotated values, and a
    # position outside the table failed closed.
    g = np.random.default_rng(13)
    T, H, Dh, R, G, P = 3, 8, 576, 64, 2, 40
    o = torch.from_numpy(g.standard_normal((T, H, Dh)).astype(np.float32) * 0.05).bfloat16()
    bits = o.view(torch.int16).numpy().view(np.uint16)
    cs = WL.rope_table(P, R).numpy()
    pos = np.array([3, 39, 40])
    codes, scales = O.inv_rope_fp8_quant(bits, pos, cs, G, R)
    hpg, D = H // G, H // G * Dh
    assert codes.shape == (G, T, D) and scales.shape == (G, T, D // 128)
    assert not codes[:, 2].any() and not scales[:, 2].any()
    of = o.float().numpy().astype(np.float64)
    for t in (0, 1):
        for gi in range(G):
            for h in range(hpg):
                head = of[t, gi * hpg + h].copy()
                th = pos[t] * 10000.0 ** (-np.arange(R // 2) * 2.0 / R)
                z = (head[Dh - R::2] + 1j * head[Dh - R + 1::2]) * np.exp(-1j * th)
                head[Dh - R::2], head[Dh - R + 1::2] = z.real, z.imag
                seg = slice(h * Dh, (h + 1) * Dh)
                dec = O.E4M3_VALUES[codes[gi, t, seg]] * np.repeat(scales[gi, t], 128)[seg]
                step = np.repeat(scales[gi, t], 128)[seg]
                err = np.abs(dec - head)
                assert (err <= np.maximum(np.abs(head) * 2.0 ** -4, step * 2.0 ** -10) + 1e-6 * np.abs(head)).all()


# --------------------------------------------------------------------------- cache write side


def test_kv_nope_encoder_matches_harness_encoder_and_floor():
    g = torch.Generator().manual_seed(17)
    x = (torch.randn(30, 512, generator=g) * torch.exp2(torch.randint(-12, 12, (30, 1), generator=g).float()))
    x[3] = 0.0
    x[4] *= 1e-9  # amax below 1e-4: the scale floors at 1e-4 / 448
    x = x.bfloat16().float()
    codes, scales = O.encode_kv_nope(x.numpy())
    hc, hs = WL.encode_fp8_rows(x)
    assert np.array_equal(codes, hc.numpy()) and np.array_equal(scales.view(np.uint32), hs.numpy().view(np.uint32))
    assert np.all(scales[3] == np.float32(np.float32(1e-4) / np.float32(448.0)))


def _kv_geom(d_nope=512, d_rope=64, block=16):
    row_b = d_nope + 2 * d_rope
    return row_b, block * (row_b + 4 * (d_nope // 64))


def test_insert_kv_rows_round_trip_and_skips():
    g = np.random.default_rng(19)
    Dn, Dr, B, npages = 512, 64, 16, 6
    row_b, page_bytes = _kv_geom(Dn, Dr, B)
    rows = torch.from_numpy(g.standard_normal((5, Dn + Dr)).astype(np.float32)).bfloat16()
    bits = rows.view(torch.int16).numpy().view(np.uint16)
    cs = WL.rope_table(100, Dr).numpy()
    pos = np.array([3, 7, 8, 50, 60])
    slots = np.array([5, -1, 17, 6 * B, 40])  # one skipped by -1, one past the pool
    before = {p: g.integers(0, 256, page_bytes).astype(np.uint8) for p in range(npages)}
    after = O.insert_kv_rows(before, bits, pos, cs, 4, slots, B, Dn, Dr, npages, page_bytes)
    back = O.dequant_rows(after, [5, 17, 40], B, Dn, Dr)
    xf = rows.float().numpy().astype(np.float64)
    for r, i in enumerate([0, 2, 4]):
        nope = O.bf16_bits_to_float(back[r, :Dn])
        assert (np.abs(nope - xf[i, :Dn]) <= np.abs(xf[i, :Dn]) * 2.0 ** -4 + 2.0 ** -9 * np.repeat(
            np.abs(xf[i, :Dn]).reshape(-1, 64).max(1), 64) / 448 * 2).all()
        cp = (pos[i] // 4) * 4
        th = cp * 10000.0 ** (-np.arange(Dr // 2) * 2.0 / Dr)
        z = (xf[i, Dn::2] + 1j * xf[i, Dn + 1::2]) * np.exp(1j * th)
        rope = O.bf16_bits_to_float(back[r, Dn:])
        assert np.allclose(rope[0::2], z.real, atol=2.0 ** -7 * np.abs(z).max())
        assert np.allclose(rope[1::2], z.imag, atol=2.0 ** -7 * np.abs(z).max())
    # only the written rows' value bytes and scale bytes changed
    for p in range(npages):
        diff = np.flatnonzero(after[p] != before[p])
        allowed = set()
        for s in (5, 17, 40):
            if s // B == p:
                o = s % B
                allowed |= set(range(o * row_b, (o + 1) * row_b))
                allowed |= set(range(B * row_b + o * 32, B * row_b + o * 32 + 32))
        assert set(diff.tolist()) <= allowed


def test_compressed_position_groups_tokens():
    assert list(O.compressed_position([0, 3, 4, 7, 8, 127, 128], 4)) == [0, 0, 4, 4, 8, 124, 128]
    assert list(O.compressed_position([5, 130], 128)) == [0, 128]
    Dn, Dr, B = 128, 32, 16
    row_b, page_bytes = _kv_geom(Dn, Dr, B)
    row = torch.randn(1, Dn + Dr, generator=torch.Generator().manual_seed(1)).bfloat16()
    bits = np.repeat(row.view(torch.int16).numpy().view(np.uint16), 3, axis=0)
    cs = WL.rope_table(64, Dr).numpy()
    out = O.insert_kv_rows({}, bits, [8, 11, 12], cs, 4, [0, 1, 2], B, Dn, Dr, 1, page_bytes)[0]
    r0, r1, r2 = (out[i * row_b: (i + 1) * row_b] for i in range(3))
    assert np.array_equal(r0, r1) and not np.array_equal(r0[Dn:], r2[Dn:])


def test_insert_index_keys_matches_the_rotated_key():
    # The written key decodes to the RoPE'd (at the compressed position), rotated key
    # within the MXFP4 step, in the right page row, with its exponents after the values.
    g = np.random.default_rng(23)
    D, R, B, npages = 128, 64, 16, 3
    page_bytes = B * (D // 2 + D // 32)
    keys = torch.from_numpy(g.standard_normal((3, D)).astype(np.float32)).bfloat16()
    bits = keys.view(torch.int16).numpy().view(np.uint16)
    cs = WL.rope_table(200, R).numpy()
    pos, slots = np.array([9, 100, 150]), np.array([3, 20, -1])
    pages = O.insert_index_keys({}, bits, pos, cs, 4, slots, B, D, npages, page_bytes)
    assert set(pages) == {0, 1}
    got, valid = O.read_index_keys(pages, np.array([0, 1]), 21, B, D, npages)
    kf = keys.float().numpy().astype(np.float64)
    import scipy.linalg
    H = scipy.linalg.hadamard(D) / np.sqrt(D)
    for i, s in ((0, 3), (1, 20)):
        cp = (pos[i] // 4) * 4
        th = cp * 10000.0 ** (-np.arange(R // 2) * 2.0 / R)
        k = kf[i].copy()
        z = (k[D - R::2] + 1j * k[D - R + 1::2]) * np.exp(1j * th)
        k[D - R::2], k[D - R + 1::2] = z.real, z.imag
        ideal = H @ k
        step = np.repeat(np.ldexp(1.0, pages[s // B][B * D // 2 + (s % B) * 4: B * D // 2 + (s % B) * 4 + 4]
                                  .astype(np.int64) - 127), 32)
        assert (np.abs(got[s] - ideal) <= step + 2.0 ** -7 * np.abs(ideal)).all()


def test_native_kv_encoder_matches_harness_and_round_trips():
    # The oracle's native writer rule against the harness's separately written one (torch
    # ops of the pages' formula), and write -> read through the pinned native reader:
    # power-of-two scales make every block's largest value land on a binade of e4m3.
    g = torch.Generator().manual_seed(29)
    x = (torch.randn(12, 448, generator=g) * torch.exp2(torch.randint(-20, 20, (12, 1), generator=g).float()))
    x[2] = 0.0
    x = x.bfloat16().float()
    codes, sb = O.encode_kv_nope_ue8m0(x.numpy())
    hc, hs = WL.encode_fp8_rows_ue8m0(x)
    assert np.array_equal(codes, hc.numpy()) and np.array_equal(sb, hs.numpy())
    B, Dn, Dr = 16, 448, 64
    page_bytes = B * (Dn + 2 * Dr + 8)
    rows = torch.cat([x, torch.randn(12, Dr, generator=g)], 1).bfloat16()
    bits = rows.view(torch.int16).numpy().view(np.uint16)
    cs = WL.rope_table(8, Dr).numpy()
    pages = O.insert_kv_rows({}, bits, [0] * 12, cs, 4, list(range(12)), B, Dn, Dr, 1, page_bytes, "ue8m0")
    back = O.bf16_bits_to_float(O.dequant_rows(pages, list(range(12)), B, Dn, Dr, "ue8m0"))
    xf = x.numpy().astype(np.float64)
    sc = np.repeat(np.ldexp(1.0, sb[:, :7].astype(np.int64) - 127), 64, axis=1)
    assert (np.abs(back[:, :Dn] - xf) <= np.maximum(np.abs(xf) * 2.0 ** -4, sc * 2.0 ** -10)).all()
    assert np.array_equal(back[:, Dn:], rows[:, Dn:].float().numpy())  # position 0: rope is the identity
