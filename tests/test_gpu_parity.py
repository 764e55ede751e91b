"""GPU parity: every step of the HIP path, called through the C ABI, against the CPU
oracle on the same seeded input bytes.

Bars: bit-exact for sparse_indices, lens and dequantized rows; top-k sets equal except
swaps among scores within 1e-5 relative of the oracle's k-th score; indexer logits
within 1e-5 relative (the per-head dots are exact, only the fp32 head sum rounds);
attention output within max-abs 5e-3 (bf16 out, fp32 accumulate) and lse within 1e-3.
Where one bf16 ulp of the exact output exceeds 5e-3 (|o| >= 1, e.g. a token that
attends to one row, so o = x), the output format alone cannot meet 5e-3 and the bar
there is one bf16 ulp of the oracle value.
The "peaky" variant (queries x4) drives outputs towards one or two rows with |x| up to
~4: there one bf16 rounding of a probability (2^-9 relative, as the PV MFMA takes
bf16 operands) or of the output (2^-9 |o|) alone exceeds 5e-3.  It is reported
(max-abs, relative RMS) and held to 5e-3 + 2^-8 * sum_j p_j |x_j|, the bound of one
bf16 rounding of every weight plus one of the output.
"""

import numpy as np
import pytest
import torch

import sparse_attention_decode_build_amd as sad
from oracle import sad_oracle as O
from sparse_attention_decode_build_amd import workloads as WL

from gpu_helpers import (bf16_to_f64, check_topk, free, gpu_attention, gpu_build, gpu_indexer, log,
                         oracle_attention, oracle_build, oracle_topk, sample_tokens)

pytestmark = pytest.mark.gpu

ATOL_OUT = 5e-3
ATOL_LSE = 1e-3

EDGE = WL.Config(
    name="edge", seed=5, window=32, ratio=4, topk=16, heads=16, d_nope=128, d_rope=32, idx_heads=4,
    idx_dim=64, block=16, idx_block=16,
    # p=0 (n_c=0); n_c=0; n_c=1; a 40-token prefill from position 0 with replay 10;
    # a decode whose window is clipped to one position; a longer decode
    groups=((1, 1, 1, 0), (1, 1, 3, 0), (1, 1, 4, 0), (1, 40, 40, 10), (1, 1, 100, 99), (1, 1, 300, 0)),
    swa_backing="all",
)

# Contexts past 64K positions (131072, 100003 and 96000): more than 16384 compressed rows,
# so the top-k kernel runs with 32 keys per thread; the middle one leaves a ragged tail.
LONG = WL.with_overrides(WL.CONFIGS["b32_8k"], name="long_ctx",
                         groups=((1, 1, 131072, 0), (1, 1, 100003, 0), (1, 1, 96000, 0)))


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sad.load()
    torch.manual_seed(0)
    yield
    torch.cuda.synchronize()


def _wl(cfg, **kw):
    log(f"[case] workload {cfg if isinstance(cfg, str) else cfg.name} {kw}")
    return WL.make_workload(cfg, "cuda", **kw)


def _full_check(wl, view, tokens, sink=None, check_gather=True, bf16_ulp_allowance=False):
    """Indexer/top-k, index build, gather and attention of `tokens` vs the oracle."""
    cfg = wl.cfg
    T = wl.num_tokens
    torch.cuda.synchronize()
    # ---- indexer + top-k
    if not cfg.dense:
        log("[step] indexer_score_topk")
        topk_g, logits = gpu_indexer(wl)
        torch.cuda.synchronize()
        topk_g = topk_g.cpu().numpy()
        logits = logits.cpu().numpy()
        tk_o, scores = oracle_topk(wl, view, tokens)
        swaps = 0
        for i, t in enumerate(tokens):
            sc, valid = scores[i]
            n = sc.shape[0]
            lg = logits[t, :n]
            assert np.all(np.isneginf(lg[~valid])), "invalid rows must score -inf"
            if valid.any():
                ref = sc[valid]
                scale = max(np.abs(ref).max(), 1e-30)
                assert np.max(np.abs(lg[valid] - ref)) <= 1e-5 * scale, f"logits token {t}"
            swaps += check_topk(topk_g[t], sc, valid, cfg.topk)
        log(f"[ok] indexer/top-k on {len(tokens)} tokens, {swaps} near-tie swaps")
        # oracle top-k for every token feeds the index build (tokens not sampled get
        # the GPU-independent oracle result too when cheap)
        tk_full = np.full((T, cfg.topk), -1, np.int32)
        tk_full[tokens] = tk_o
    else:
        tk_full = None
    # ---- build_sparse_indices on the oracle's top-k: bit-exact
    log("[step] build_sparse_indices")
    tk_dev = torch.from_numpy(tk_full).cuda() if tk_full is not None else None
    si_g, lens_g = gpu_build(wl, tk_dev)
    torch.cuda.synchronize()
    si_o, lens_o = oracle_build(wl, view, tk_full, tokens=tokens)
    assert np.array_equal(si_g.cpu().numpy()[tokens], si_o)
    assert np.array_equal(lens_g.cpu().numpy()[tokens], lens_o)
    log("[ok] build_sparse_indices bit-exact")
    si_full = np.full((T, si_o.shape[1]), -1, np.int32)
    lens_full = np.zeros(T, np.int32)
    si_full[tokens] = si_o
    lens_full[tokens] = lens_o
    # ---- gather + dequant: bit-exact
    if check_gather:
        log("[step] gather_dequant_kv")
        kv, _ = _caches(wl)
        sub = tokens[: min(len(tokens), 16)]
        si_sub = si_g[torch.as_tensor(sub, device="cuda")].contiguous()
        lens_sub = lens_g[torch.as_tensor(sub, device="cuda")].contiguous()
        rows_g = sad.gather_dequant_kv(kv, kv, si_sub, lens_sub, cfg.window, wl.padded_topk)
        torch.cuda.synchronize()
        rows_o = O.gather_dequant(view.kv_pages, view.kv_pages, si_o[: len(sub)], lens_o[: len(sub)],
                                  cfg.window, cfg.block, cfg.block, cfg.d_nope, cfg.d_rope, cfg.kv_format)
        got = rows_g.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, rows_o)
        log(f"[ok] gather_dequant_kv bit-exact on {len(sub)} tokens")
    # ---- attention on the (bit-identical) index rows
    log("[step] sparse_mla_decode")
    sink_dev = None if sink is None else torch.from_numpy(sink.astype(np.float32)).cuda()
    out_g, lse_g = gpu_attention(wl, si_g, lens_g, sink=sink_dev, with_lse=True)
    torch.cuda.synchronize()
    o_o, lse_o, mass = oracle_attention(wl, view, si_full, lens_full, tokens, sink=sink, return_mass=True)
    got = bf16_to_f64(out_g)[tokens]
    err = np.abs(got - o_o)
    rms = float(np.sqrt(np.mean((got - o_o) ** 2)) / max(np.sqrt(np.mean(o_o ** 2)), 1e-30))
    log(f"[report] attention max-abs {err.max():.3e} rel-rms {rms:.3e} max|o| {np.abs(o_o).max():.3f}")
    tol = np.maximum(ATOL_OUT, _bf16_ulp(o_o)) + (2.0 ** -8 * mass if bf16_ulp_allowance else 0.0)
    assert np.all(err <= tol)
    lg = lse_g.cpu().numpy()[tokens]
    fin = np.isfinite(lse_o)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.max(np.abs(lg[fin] - lse_o[fin]), initial=0.0) <= ATOL_LSE
    return si_g, lens_g, out_g


def _bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def _caches(wl):
    cfg = wl.cfg
    return (sad.KvCache(wl.kv_pool, cfg.block, cfg.d_nope, cfg.d_rope, WL.kv_scale_format(cfg)),
            sad.IndexerCache(wl.idx_pool, cfg.idx_block, cfg.idx_dim))


# ---------------------------------------------------------------------------- small


@pytest.mark.parametrize("name", ["tiny", "b32_8k", "tiny_native", "b32_8k_native"])
def test_small_config_every_step(name):
    wl = _wl(name)
    view = WL.host_view(wl)
    _full_check(wl, view, list(range(wl.num_tokens)))
    free(wl)


def test_tiny_sparse_equals_dense_selfcheck():
    cfg = WL.with_overrides(WL.CONFIGS["tiny"], window=256, topk=64)
    wl = _wl(cfg)
    view = WL.host_view(wl)
    _, lens, out = _full_check(wl, view, [0])
    assert int(lens[0]) == 64


@pytest.mark.parametrize("name", ["tiny", "b32_8k", "tiny_native"])
def test_peaky_queries(name):
    wl = _wl(name, q_scale=4.0)
    view = WL.host_view(wl)
    _full_check(wl, view, list(range(wl.num_tokens)), check_gather=False, bf16_ulp_allowance=True)
    free(wl)


def test_attention_sink_and_lse():
    wl = _wl("tiny")
    view = WL.host_view(wl)
    rng = np.random.default_rng(11)
    sink = rng.standard_normal(wl.cfg.heads) * 2.0
    _full_check(wl, view, [0], sink=sink, check_gather=False)


def test_edge_batch():
    wl = _wl(EDGE)
    view = WL.host_view(wl)
    _full_check(wl, view, list(range(wl.num_tokens)))
    free(wl)


@pytest.mark.parametrize("heads,requests", [(40, 256), (72, 128), (96, 128), (120, 128), (72, 4), (120, 3)])
def test_head_counts_with_partial_head_groups(heads, requests):
    """Head counts whose last group of 64 heads is partial: a head block with absent
    heads (40, 72, 120) or an idle one (96).  With 256 or more (token, head group)
    pairs one workgroup covers a token's columns and stages O through LDS; with a few
    tokens the columns are split and merged.  The rows after the output are untouched."""
    cfg = WL.with_overrides(WL.CONFIGS["b32_8k"], name=f"h{heads}_r{requests}", heads=heads,
                            groups=((requests, 1, 512, 0),))
    wl = _wl(cfg)
    view = WL.host_view(wl)
    tokens = list(range(0, wl.num_tokens, max(1, wl.num_tokens // 24)))
    si, lens, out = _full_check(wl, view, tokens, check_gather=False)
    # the same launch into a buffer with a guard region after the output
    T, H, D = out.shape
    guard = 4096
    buf = torch.full((T * H * D + guard,), -7, dtype=torch.int16, device="cuda")
    kv, _ = _caches(wl)
    out2 = buf[: T * H * D].view(torch.bfloat16).view(T, H, D)
    sad.sparse_mla_decode(wl.layers[0].q, kv, kv, si, lens, cfg.window, wl.padded_topk, wl.softmax_scale,
                          out=out2)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16)), "same launch, same bits"
    assert bool((buf[T * H * D:] == -7).all()), "a store past the output"
    free(wl)


def test_long_context_32_keys_per_thread():
    wl = _wl(LONG)
    view = WL.host_view(wl)
    assert wl.layers[0].idx_bt.shape[1] * wl.cfg.idx_block > 16 * 1024
    _full_check(wl, view, list(range(wl.num_tokens)), check_gather=False)
    free(wl)


@pytest.mark.parametrize("base,idx_dim,idx_block", [("tiny", 128, 16), ("b32_8k", 64, 64)])
def test_indexer_key_dim_and_page_size(base, idx_dim, idx_block):
    """The scoring kernel's other two (key dim, rows per page) forms: 128 x 16 and 64 x 64."""
    cfg = WL.with_overrides(WL.CONFIGS[base], name=f"{base}_i{idx_dim}_b{idx_block}", idx_dim=idx_dim,
                            idx_block=idx_block)
    if base == "b32_8k":
        cfg = WL.with_overrides(cfg, groups=((6, 1, 8192, 0),))
    wl = _wl(cfg)
    view = WL.host_view(wl)
    _full_check(wl, view, list(range(wl.num_tokens)), check_gather=False)
    free(wl)


def test_edge_fail_closed_tables():
    """Unbacked pages, ids past the pool and random local ids (incl. -1 and >= n_c)."""
    wl = _wl(EDGE)
    cfg = wl.cfg
    L = wl.layers[0]
    g = torch.Generator(device="cpu").manual_seed(3)
    holes = torch.rand(L.swa_bt.shape, generator=g) < 0.2
    L.swa_bt[holes.cuda()] = -1
    holes = torch.rand(L.comp_bt.shape, generator=g) < 0.2
    L.comp_bt[holes.cuda()] = -1
    L.comp_bt[0, 0] = wl.kv_pool.shape[0] + 3  # past the pool
    view = WL.host_view(wl)
    T = wl.num_tokens
    tk = torch.randint(-3, 80, (T, cfg.topk + 5), generator=g, dtype=torch.int32)
    si_g, lens_g = sad.build_sparse_indices(
        wl.query_start_loc, wl.seq_lens, wl.token_to_req, wl.replay_start, L.swa_bt, cfg.block,
        wl.kv_pool.shape[0], L.comp_bt, cfg.block, wl.kv_pool.shape[0], tk.cuda(), cfg.topk,
        cfg.window, cfg.ratio, wl.padded_topk)
    torch.cuda.synchronize()
    si_o, lens_o = oracle_build(wl, view, tk.numpy())
    assert np.array_equal(si_g.cpu().numpy(), si_o)
    assert np.array_equal(lens_g.cpu().numpy(), lens_o)
    # attention over rows with holes
    out_g, _ = gpu_attention(wl, si_g, lens_g)
    torch.cuda.synchronize()
    o_o, _ = oracle_attention(wl, view, si_o, lens_o, list(range(T)))
    assert np.all(np.abs(bf16_to_f64(out_g) - o_o) <= np.maximum(ATOL_OUT, _bf16_ulp(o_o)))


def test_nothing_attended_gives_zero_and_neg_inf_lse():
    wl = _wl("tiny")
    cfg = wl.cfg
    T = wl.num_tokens
    si = torch.full((T, cfg.window + wl.padded_topk), -1, dtype=torch.int32, device="cuda")
    lens = torch.zeros(T, dtype=torch.int32, device="cuda")
    out, lse = gpu_attention(wl, si, lens, with_lse=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    assert torch.all(torch.isneginf(lse)).item()


@pytest.mark.parametrize("window,padded", [(3, 2), (0, 5), (7, 0), (0, 0), (5, 64)])
def test_narrow_index_rows(window, padded):
    """Index rows narrower than one wave's 8 slot ids (and an empty row)."""
    wl = _wl("tiny")
    cfg = wl.cfg
    view = WL.host_view(wl)
    T = wl.num_tokens
    rng = np.random.default_rng(window * 100 + padded)
    pages = np.array(sorted(view.kv_pages.keys()), np.int64)  # pages the host view holds
    si = (rng.choice(pages, (T, window + padded)) * cfg.block
          + rng.integers(0, cfg.block, (T, window + padded))).astype(np.int32)
    si[rng.random(si.shape) < 0.2] = -1
    lens = rng.integers(0, padded + 1, T).astype(np.int32)
    kv, _ = _caches(wl)
    L = wl.layers[0]
    lse = torch.empty((T, cfg.heads), dtype=torch.float32, device="cuda")
    out = sad.sparse_mla_decode(L.q, kv, kv, torch.from_numpy(si).cuda(), torch.from_numpy(lens).cuda(),
                                window, padded, wl.softmax_scale, lse=lse)
    torch.cuda.synchronize()
    o_o, lse_o = O.sparse_mla_decode(view.q, view.kv_pages, view.kv_pages, si, lens, window, cfg.block,
                                     cfg.block, cfg.d_nope, cfg.d_rope, wl.softmax_scale,
                                     tokens=list(range(T)))
    err = np.abs(bf16_to_f64(out) - o_o)
    assert np.all(err <= np.maximum(ATOL_OUT, _bf16_ulp(o_o)))
    lg = lse.cpu().numpy()
    fin = np.isfinite(lse_o)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.max(np.abs(lg[fin] - lse_o[fin]), initial=0.0) <= ATOL_LSE


def test_empty_batch_is_a_no_op():
    wl = _wl("tiny")
    cfg = wl.cfg
    e32 = torch.empty(0, dtype=torch.int32, device="cuda")
    L = wl.layers[0]
    si, lens = sad.build_sparse_indices(torch.zeros(1, dtype=torch.int32, device="cuda"), e32, e32, None,
                                        L.swa_bt[:0], cfg.block, 1, L.comp_bt[:0], cfg.block, 1, None, 0,
                                        cfg.window, cfg.ratio, wl.padded_topk)
    assert si.shape == (0, cfg.window + wl.padded_topk)
    kv, _ = _caches(wl)
    out = sad.sparse_mla_decode(L.q[:0], kv, kv, si, lens, cfg.window, wl.padded_topk, 0.1)
    assert out.shape[0] == 0


def test_dequant_every_e4m3_code_bit_exact():
    """A page whose rows hold every finite e4m3 byte, with assorted fp32 scales."""
    cfg = WL.CONFIGS["tiny"]
    B, Dn, Dr = cfg.block, cfg.d_nope, cfg.d_rope
    rowb = Dn + 2 * Dr
    codes = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)  # 254 finite codes
    page = np.zeros(cfg.kv_page_bytes, np.uint8)
    rng = np.random.default_rng(2)
    for o in range(B):
        page[o * rowb: o * rowb + Dn] = np.roll(np.resize(codes, Dn), 7 * o)
        page[o * rowb + Dn: (o + 1) * rowb] = rng.integers(0, 256, 2 * Dr, dtype=np.uint8) & 0x3F
        sc = (rng.random(Dn // 64) * 3 + 1e-3).astype(np.float32) * np.float32(2.0 ** (o - 8))
        page[B * rowb + o * 4 * (Dn // 64): B * rowb + (o + 1) * 4 * (Dn // 64)] = sc.view(np.uint8)
    pool = torch.from_numpy(np.stack([page, page])).cuda()
    kv = sad.KvCache(pool, B, Dn, Dr)
    si = torch.tensor([[B + o for o in range(B)] + [-1] * 16], dtype=torch.int32, device="cuda")
    W = B
    lens = torch.tensor([0], dtype=torch.int32, device="cuda")
    got = sad.gather_dequant_kv(kv, kv, si, lens, W, 16)
    torch.cuda.synchronize()
    want = O.gather_dequant({1: page}, {1: page}, si.cpu().numpy(), [0], W, B, B, Dn, Dr)
    assert np.array_equal(got.view(torch.int16).cpu().numpy().view(np.uint16), want)


def test_deterministic():
    wl = _wl("b32_8k")
    topk_a, _ = gpu_indexer(wl, logits=False)
    topk_b, _ = gpu_indexer(wl, logits=False)
    si_a, lens_a = gpu_build(wl, topk_a)
    out_a, _ = gpu_attention(wl, si_a, lens_a)
    out_b, _ = gpu_attention(wl, si_a, lens_a)
    torch.cuda.synchronize()
    assert torch.equal(topk_a, topk_b)
    assert torch.equal(out_a.view(torch.int16), out_b.view(torch.int16))
    free(wl)


# ---------------------------------------------------------------------------- full size


@pytest.mark.slow
def test_b128_64k_full_size_sampled():
    """128 requests at 64K context over a ~196 GB pool: all tokens run on the GPU in
    the benchmark's launch configuration; index rows are compared on every token and
    the oracle recomputes scores, top-k, rows and attention for sampled tokens."""
    wl = _wl("b128_64k")
    tokens = [0, 17, 63, 127]
    view = WL.host_view(wl, reqs=tokens)
    all_view = view
    _full_check(wl, all_view, tokens)
    free(wl)


@pytest.mark.slow
def test_b128_64k_native_record_full_size_sampled():
    """The pages' native KV record (448 fp8 + 64 bf16, ue8m0 scales) at 128 requests x
    64K context over a ~170 GB pool, in the benchmark's launch configuration."""
    wl = _wl("b128_64k_native")
    tokens = [0, 45, 127]
    view = WL.host_view(wl, reqs=tokens)
    _full_check(wl, view, tokens)
    free(wl)


@pytest.mark.slow
def test_mixed_batch_sampled():
    wl = _wl("mixed")
    tokens = sample_tokens(wl, n_decode=4, n_prefill=8)
    reqs = sorted(set(wl.token_to_req.cpu().numpy()[tokens].tolist()))
    view = WL.host_view(wl, reqs=reqs)
    _full_check(wl, view, tokens)
    free(wl)


@pytest.mark.slow
def test_dense_1m_full():
    wl = _wl("dense_1m")
    view = WL.host_view(wl)
    _full_check(wl, view, list(range(wl.num_tokens)))
    free(wl)


@pytest.mark.parametrize("name", ["tiny", "b32_8k", "edge", "edge_holes", "b128_64k", "long_ctx"])
def test_fused_indexer_and_index_build_equal_the_two_calls(name):
    # indexer_topk_sparse_indices is defined as indexer_score_topk then build_sparse_indices:
    # all three outputs bit-identical to the two-call path (with holes in both block tables
    # and a page past the pool in the "edge_holes" case).
    cfg = EDGE if name.startswith("edge") else LONG if name == "long_ctx" else name
    wl = _wl(cfg)
    c = wl.cfg
    L0 = wl.layers[0]
    if name == "edge_holes":
        g = torch.Generator(device="cpu").manual_seed(7)
        L0.swa_bt[(torch.rand(L0.swa_bt.shape, generator=g) < 0.2).cuda()] = -1
        L0.comp_bt[(torch.rand(L0.comp_bt.shape, generator=g) < 0.2).cuda()] = -1
        L0.comp_bt[0, 0] = wl.kv_pool.shape[0] + 3
    _, idx = _caches(wl)
    n_pages = wl.kv_pool.shape[0]
    tk_a, _ = gpu_indexer(wl, logits=False)
    si_a, lens_a = gpu_build(wl, tk_a)
    tk_b, si_b, lens_b = sad.indexer_topk_sparse_indices(
        wl.query_start_loc, wl.seq_lens, wl.token_to_req, L0.idx_q_values, L0.idx_q_scales, L0.idx_weights, idx,
        L0.idx_bt, c.ratio, c.topk, wl.replay_start, L0.swa_bt, c.block, n_pages, L0.comp_bt, c.block, n_pages,
        c.window, wl.padded_topk)
    torch.cuda.synchronize()
    assert torch.equal(tk_a, tk_b)
    assert torch.equal(si_a, si_b)
    assert torch.equal(lens_a, lens_b)
    free(wl)
