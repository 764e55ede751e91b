"""GPU parity: every step of the HIP path, called through the C ABI, against the CPU
oracle on the same seeded input bytes.

Bars:
- sparse_indices and lens: bit-exact on every token, built from the GPU's own top-k (the
  build is a function of the top-k row, so the two sides see the same input);
- dequantized rows: bit-exact;
- top-k: sets equal to the oracle's except swaps among scores within 1e-5 relative of
  the oracle's k-th score; indexer logits within 1e-5 relative (the per-head dots are
  exact, only the fp32 head sum rounds);
- attention output: max(5e-3, half an ulp of the bf16 output + 2^-8 (1 + 2^-6) spread +
  2^-11 (|o| + spread)) per element, spread = sum_j p_j |x_j - o| (see
  gpu_helpers.check_attention): beyond the bf16 rounding of the output, the PV MFMA takes
  every softmax weight rounded to bf16, which moves o by at most 2^-8 spread (bf16's unit roundoff).  Each case
  reports how many elements exceed the plain 5e-3; lse within 1e-3.
The "peaky" variant (queries x4) concentrates the weights on a few rows (|x| up to ~4),
where the weight rounding is the largest term; it is reported separately.
"""

import numpy as np
import pytest
import torch

import sparse_attention_decode_build_amd as sad
from oracle import sad_oracle as O
from sparse_attention_decode_build_amd import workloads as WL

from gpu_helpers import (ATOL_LSE, bf16_to_f64, check_attention, check_topk, free, gpu_attention, gpu_build,
                         gpu_fused, gpu_indexer, kv_caches, log, oracle_attention, oracle_build, oracle_gather,
                         oracle_topk, sample_tokens)

pytestmark = pytest.mark.gpu

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


def _full_check(wl, view, tokens, sink=None, check_gather=True, label=None):
    """Every step vs the oracle: indexer logits and top-k on `tokens`; the index build on
    every token (from the GPU's own top-k), and the fused indexer + build call equal to
    the two calls on every token; gather on up to 16 of `tokens`; attention on `tokens`."""
    cfg = wl.cfg
    label = label or cfg.name
    T = wl.num_tokens
    torch.cuda.synchronize()
    topk_dev = None
    # ---- indexer + top-k
    if not cfg.dense:
        log("[step] indexer_score_topk")
        topk_dev, logits = gpu_indexer(wl)
        torch.cuda.synchronize()
        topk_g = topk_dev.cpu().numpy()
        logits = logits.cpu().numpy()
        _, scores = oracle_topk(wl, view, tokens)
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
    # ---- build_sparse_indices on the GPU's top-k: bit-exact on every token
    log("[step] build_sparse_indices")
    si_g, lens_g = gpu_build(wl, topk_dev)
    torch.cuda.synchronize()
    si_o, lens_o = oracle_build(wl, view, topk_dev.cpu().numpy() if topk_dev is not None else None)
    si_np, lens_np = si_g.cpu().numpy(), lens_g.cpu().numpy()
    assert np.array_equal(si_np, si_o), "sparse_indices differ from the oracle"
    assert np.array_equal(lens_np, lens_o), "sparse_topk_lens differ from the oracle"
    log(f"[ok] build_sparse_indices bit-exact on all {T} tokens")
    # ---- the fused call: the same three outputs, bit for bit, on every token
    if not cfg.dense:
        log("[step] indexer_topk_sparse_indices")
        tk_f, si_f, lens_f = gpu_fused(wl)
        torch.cuda.synchronize()
        assert torch.equal(tk_f, topk_dev) and torch.equal(si_f, si_g) and torch.equal(lens_f, lens_g)
        log("[ok] fused indexer + index build equal to the two calls")
    # ---- gather + dequant: bit-exact
    if check_gather:
        log("[step] gather_dequant_kv")
        swa, comp = kv_caches(wl)
        sub = tokens[: min(len(tokens), 16)]
        sub_dev = torch.as_tensor(sub, device="cuda")
        rows_g = sad.gather_dequant_kv(swa, comp, si_g[sub_dev].contiguous(), lens_g[sub_dev].contiguous(),
                                       cfg.window, wl.padded_topk)
        torch.cuda.synchronize()
        rows_o = oracle_gather(wl, view, si_o[sub], lens_o[sub])
        assert np.array_equal(rows_g.view(torch.int16).cpu().numpy().view(np.uint16), rows_o)
        log(f"[ok] gather_dequant_kv bit-exact on {len(sub)} tokens")
    # ---- attention on the (bit-identical) index rows
    log("[step] sparse_mla_decode")
    sink_dev = None if sink is None else torch.from_numpy(sink.astype(np.float32)).cuda()
    out_g, lse_g = gpu_attention(wl, si_g, lens_g, sink=sink_dev, with_lse=True)
    torch.cuda.synchronize()
    o_o, lse_o = oracle_attention(wl, view, si_o, lens_o, tokens, sink=sink)
    got = bf16_to_f64(out_g)[tokens]
    check_attention(wl, view, tokens, got, o_o, si_o, lens_o, sink=sink, label=label)
    lg = lse_g.cpu().numpy()[tokens]
    fin = np.isfinite(lse_o)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.max(np.abs(lg[fin] - lse_o[fin]), initial=0.0) <= ATOL_LSE
    return si_g, lens_g, out_g


# ---------------------------------------------------------------------------- small


@pytest.mark.parametrize("name", ["tiny", "b32_8k", "tiny_native", "b32_8k_native", "two_cache_tiny",
                                  "two_cache_b8_8k"])
def test_small_config_every_step(name):
    """Every step on every token.  The two_cache_* workloads keep the window rows in a pool
    of their own with 64-row pages and the compressed rows in 16-row pages ([backend]
    forward_deepseek_v4_decode: k_cache / extra_k_cache), so the index build maps the two
    segments through different page sizes and the gather and attention read two pools."""
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


@pytest.mark.parametrize("name", ["tiny", "b32_8k", "tiny_native", "two_cache_tiny"])
def test_peaky_queries(name):
    wl = _wl(name, q_scale=4.0)
    view = WL.host_view(wl)
    _full_check(wl, view, list(range(wl.num_tokens)), check_gather=False, label=f"{name} peaky")
    free(wl)


@pytest.mark.parametrize("requests", [8, 256])
def test_lazy_rescale_under_very_peaky_queries(requests):
    # queries x16: log2-unit logits span about +-100, so a 32-column tile's maximum
    # passes the running maximum by more than the 2^8 slack on about 8% of the tiles
    # (about 1% at x4, never at x1, counted on the CPU from the oracle's rows) and the O
    # accumulators are rescaled often (split with 8 requests, unsplit with 256)
    cfg = WL.with_overrides(WL.CONFIGS["b32_8k"], name=f"b32_8k_q16_r{requests}", groups=((requests, 1, 2048, 0),))
    wl = _wl(cfg, q_scale=16.0)
    view = WL.host_view(wl)
    tokens = list(range(0, wl.num_tokens, max(1, wl.num_tokens // 16)))
    _full_check(wl, view, tokens, check_gather=False, label=f"{cfg.name} peaky")
    free(wl)


@pytest.mark.parametrize("base,requests,native", [("tiny", 0, False), ("b32_8k", 0, False),
                                                 ("b32_8k", 256, False), ("b32_8k", 8, True),
                                                 ("b32_8k", 256, True)])
def test_attention_sink_and_lse(base, requests, native):
    # a per-head sink: in the kernel's epilogue when one workgroup covers a token's
    # columns (256 requests of one head group), in the combine when they are split
    over = dict(d_nope=448, kv_format="ue8m0") if native else {}
    if requests:
        over["groups"] = ((requests, 1, 2048, 0),)
    cfg = WL.with_overrides(WL.CONFIGS[base], name=f"{base}_sink_r{requests}{'_native' if native else ''}", **over)
    wl = _wl(cfg)
    view = WL.host_view(wl)
    rng = np.random.default_rng(11)
    sink = rng.standard_normal(wl.cfg.heads) * 2.0
    tokens = list(range(0, wl.num_tokens, max(1, wl.num_tokens // 16)))
    _full_check(wl, view, tokens, sink=sink, check_gather=False)
    free(wl)


def test_edge_batch():
    wl = _wl(EDGE)
    view = WL.host_view(wl)
    _full_check(wl, view, list(range(wl.num_tokens)))
    free(wl)


@pytest.mark.parametrize("heads,requests,native", [(40, 256, False), (72, 128, False), (96, 128, False),
                                                  (120, 128, False), (72, 4, False), (120, 3, False),
                                                  (72, 128, True), (120, 3, True)])
def test_head_counts_with_partial_head_groups(heads, requests, native):
    """Head counts whose last group of 64 heads is partial: a head block with absent
    heads (40, 72, 120) or an idle one (96).  With many (token, head group) pairs one
    workgroup covers a token's columns; with a few tokens the columns are split and
    merged.  The rows after the output are untouched.  Also for the native record."""
    over = dict(d_nope=448, kv_format="ue8m0") if native else {}
    cfg = WL.with_overrides(WL.CONFIGS["b32_8k"], name=f"h{heads}_r{requests}{'_native' if native else ''}",
                            heads=heads, groups=((requests, 1, 512, 0),), **over)
    wl = _wl(cfg)
    view = WL.host_view(wl)
    tokens = list(range(0, wl.num_tokens, max(1, wl.num_tokens // 24)))
    si, lens, out = _full_check(wl, view, tokens, check_gather=False)
    # the same launch into a buffer with a guard region after the output
    T, H, D = out.shape
    guard = 4096
    buf = torch.full((T * H * D + guard,), -7, dtype=torch.int16, device="cuda")
    swa, comp = kv_caches(wl)
    out2 = buf[: T * H * D].view(torch.bfloat16).view(T, H, D)
    sad.sparse_mla_decode(wl.layers[0].q, swa, comp, si, lens, cfg.window, wl.padded_topk, wl.softmax_scale,
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


def _punch(table, frac, seed, past_pool):
    """Set a seeded fraction of a block table's entries to -1 and one to a page past the pool."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    holes = torch.rand(table.shape, generator=g) < frac
    table[holes.to(table.device)] = -1
    table[0, 0] = past_pool


def test_edge_fail_closed_tables():
    """Unbacked pages, ids past the pool and random local ids (incl. -1 and >= n_c)."""
    wl = _wl(EDGE)
    cfg = wl.cfg
    L = wl.layers[0]
    _punch(L.swa_bt, 0.2, 3, wl.swa_pool.shape[0] + 3)
    _punch(L.comp_bt, 0.2, 4, wl.kv_pool.shape[0] + 3)
    view = WL.host_view(wl)
    T = wl.num_tokens
    g = torch.Generator(device="cpu").manual_seed(5)
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
    check_attention(wl, view, list(range(T)), bf16_to_f64(out_g), o_o, si_o, lens_o, label="edge holes")


@pytest.mark.parametrize("name", ["edge", "b32_8k", "two_cache_b8_8k"])
def test_indexer_table_holes(name):
    """Unbacked indexer key pages (-1) and a page past the indexer pool inside n_c ([ops]
    read_deepseek_v4_indexer_mxfp4_cache masks them; [backend] safe_page_ids fails closed):
    their rows score -inf, are never chosen (top-k pads with -1 when fewer than k rows are
    backed), and the fused call still equals the two calls; holes in the window and
    compressed tables too."""
    cfg = EDGE if name == "edge" else WL.with_overrides(WL.CONFIGS[name], groups=((6, 1, 8192, 0),))
    wl = _wl(cfg)
    L = wl.layers[0]
    _punch(L.idx_bt, 0.3, 9, wl.idx_pool.shape[0] + 5)
    if name == "edge":
        _punch(L.swa_bt, 0.2, 10, wl.swa_pool.shape[0] + 1)
        _punch(L.comp_bt, 0.2, 11, wl.kv_pool.shape[0] + 1)
    view = WL.host_view(wl)
    _full_check(wl, view, list(range(wl.num_tokens)), check_gather=name != "b32_8k", label=f"{name} idx holes")
    free(wl)


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
    """Index rows narrower than one tile's slot ids (and an empty row)."""
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
    swa, comp = kv_caches(wl)
    L = wl.layers[0]
    lse = torch.empty((T, cfg.heads), dtype=torch.float32, device="cuda")
    out = sad.sparse_mla_decode(L.q, swa, comp, torch.from_numpy(si).cuda(), torch.from_numpy(lens).cuda(),
                                window, padded, wl.softmax_scale, lse=lse)
    torch.cuda.synchronize()
    o_o, lse_o = O.sparse_mla_decode(view.q, view.swa_pages, view.kv_pages, si, lens, window, cfg.block,
                                     cfg.block, cfg.d_nope, cfg.d_rope, wl.softmax_scale,
                                     tokens=list(range(T)))
    check_attention(wl, view, list(range(T)), bf16_to_f64(out), o_o, si, lens, label=f"narrow {window}+{padded}",
                    window=window)
    lg = lse.cpu().numpy()
    fin = np.isfinite(lse_o)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.max(np.abs(lg[fin] - lse_o[fin]), initial=0.0) <= ATOL_LSE


@pytest.mark.parametrize("rep", [1, 8])
def test_tile_counts_and_holes_on_the_headline_row(rep):
    """The headline row (512 fp8 + 64 bf16, 64 heads) with index rows of 1 to 8 tiles per
    token: widths at tile boundaries and one off either side, fully valid rows (no
    mask to apply) and rows with -1 and past-pool ids in their tiles (masked).  With 32
    tokens the columns are split in two, so splits hold 0 to 4 tiles (the loops' first,
    steady and drain steps, and a split with nothing); with the tokens repeated 8 times
    (256 units) nothing is split.  Every token against the oracle, lse included."""
    wl = _wl("b32_8k")
    cfg = wl.cfg
    view = WL.host_view(wl)
    T0 = wl.num_tokens
    T = T0 * rep
    window, padded = 0, 256
    rng = np.random.default_rng(4242 + rep)
    pages = np.array(sorted(view.kv_pages.keys()), np.int64)
    si = (rng.choice(pages, (T, padded)) * cfg.block + rng.integers(0, cfg.block, (T, padded))).astype(np.int64)
    widths = np.array([1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 128, 129, 160, 191, 224, 256], np.int32)
    lens = widths[np.arange(T) % len(widths)].astype(np.int32)
    holes = (np.arange(T) // len(widths)) % 2 == 1  # every other round of widths has holes
    for t in np.nonzero(holes)[0]:
        m = rng.random(padded) < 0.15
        si[t, m] = -1
        past = rng.random(padded) < 0.05
        si[t, past] = (wl.kv_pool.shape[0] + 3) * cfg.block  # a page past the pool: masked
    si = si.astype(np.int32)
    # the kernel masks ids past the pool as it masks -1 (fail closed); the oracle's attention
    # takes rows whose ids are already safe, so it gets those ids as -1
    si_o = np.where(si >= wl.kv_pool.shape[0] * cfg.block, -1, si).astype(np.int32)
    q = wl.layers[0].q
    q_rep = q.repeat(rep, 1, 1).contiguous() if rep > 1 else q
    q_bits = np.tile(view.q, (rep, 1, 1)) if rep > 1 else view.q
    swa, comp = kv_caches(wl)
    lse = torch.empty((T, cfg.heads), dtype=torch.float32, device="cuda")
    out = sad.sparse_mla_decode(q_rep, swa, comp, torch.from_numpy(si).cuda(), torch.from_numpy(lens).cuda(),
                                window, padded, wl.softmax_scale, lse=lse)
    torch.cuda.synchronize()
    tokens = list(range(T)) if rep == 1 else list(range(0, T, 3))
    o_o, lse_o = O.sparse_mla_decode(q_bits, view.swa_pages, view.kv_pages, si_o, lens, window, cfg.block,
                                     cfg.block, cfg.d_nope, cfg.d_rope, wl.softmax_scale, tokens=tokens)
    got = bf16_to_f64(out[tokens])
    check_attention(wl, view, tokens, got, o_o, si_o, lens, q_bits=q_bits, label=f"tile counts x{rep}",
                    window=window)
    lg = lse.cpu().numpy()[tokens]
    fin = np.isfinite(lse_o)
    assert np.array_equal(np.isfinite(lg), fin)
    assert np.max(np.abs(lg[fin] - lse_o[fin]), initial=0.0) <= ATOL_LSE
    free(wl)


def test_empty_batch_is_a_no_op():
    wl = _wl("tiny")
    cfg = wl.cfg
    e32 = torch.empty(0, dtype=torch.int32, device="cuda")
    L = wl.layers[0]
    si, lens = sad.build_sparse_indices(torch.zeros(1, dtype=torch.int32, device="cuda"), e32, e32, None,
                                        L.swa_bt[:0], cfg.block, 1, L.comp_bt[:0], cfg.block, 1, None, 0,
                                        cfg.window, cfg.ratio, wl.padded_topk)
    assert si.shape == (0, cfg.window + wl.padded_topk)
    swa, comp = kv_caches(wl)
    out = sad.sparse_mla_decode(L.q[:0], swa, comp, si, lens, cfg.window, wl.padded_topk, 0.1)
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
@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,q_scale", [("b128_64k", 1.0), ("b128_64k_native", 1.0), ("b128_64k", 4.0)])
def test_b128_64k_full_size_every_token(name, q_scale):
    """128 requests at 64K context over a ~196 GB pool (~170 GB for the native record), in
    the benchmark's launch configuration: every token's logits, top-k, index row, fused
    call and attention output against the oracle (rows of 16 tokens for the gather).
    q_scale 4 is the peaky variant."""
    wl = _wl(name, q_scale=q_scale)
    view = WL.host_view(wl)
    _full_check(wl, view, list(range(wl.num_tokens)), label=f"{name} q x{q_scale:g}")
    free(wl)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_mixed_batch_sampled():
    """The mixed batch (64 decode tokens, then 4 prefill chunks of 4096): the index build on
    all 16,448 tokens; indexer, top-k and attention on all 64 decode tokens plus 256 seeded
    prefill tokens and every prefill token at p = 0, with a window clipped by replay_start
    or with fewer than k compressed rows."""
    wl = _wl("mixed")
    tokens = sample_tokens(wl, n_decode=64, n_prefill=256)
    log(f"[case] mixed: {len(tokens)} sampled tokens")
    view = WL.host_view(wl)
    _full_check(wl, view, tokens)
    free(wl)


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_csa_1m_top_k_past_one_workgroup():
    """262144 compressed rows per token (1M context at ratio 4): the top-k runs in 8
    chunks whose candidates are merged; every step on all 4 tokens vs the oracle."""
    wl = _wl("csa_1m")
    view = WL.host_view(wl)
    _full_check(wl, view, list(range(wl.num_tokens)))
    free(wl)


def test_native_record_two_caches():
    # the pages' native record (448 + 64, ue8m0) in the two-cache form: window pages of 64
    # rows and compressed pages of 16 rows in pools of their own (the dim-split kernel's
    # two-cache native instantiation), 3 requests, so the columns are split as well
    cfg = WL.with_overrides(WL.CONFIGS["two_cache_b8_8k"], name="two_cache_b3_8k_native", d_nope=448,
                            kv_format="ue8m0", groups=((3, 1, 8192, 0),))
    wl = _wl(cfg)
    view = WL.host_view(wl)
    _full_check(wl, view, list(range(wl.num_tokens)))
    free(wl)


@pytest.mark.parametrize("base,native", [("two_cache_b8_8k", False), ("two_cache_b8_8k", True),
                                         ("b32_8k", True)])
def test_unsplit_with_and_without_lse(base, native):
    # 256 requests of one 64-head group fill the GPU without column splits, so the
    # kernels run in their one-pass form; asked without lse they must give the same
    # output, bit for bit, as asked with it (which is checked against the oracle)
    over = dict(d_nope=448, kv_format="ue8m0") if native else {}
    cfg = WL.with_overrides(WL.CONFIGS[base], name=f"{base}_b256_2k{'_native' if native else ''}",
                            groups=((256, 1, 2048, 0),), **over)
    wl = _wl(cfg)
    c = wl.cfg
    assert sad.sparse_mla_decode_workspace_size(wl.num_tokens, c.heads, c.window + wl.padded_topk, c.dqk) == 0
    view = WL.host_view(wl)
    si_g, lens_g, out_lse = _full_check(wl, view, list(range(wl.num_tokens)), check_gather=False)
    out_nolse, _ = gpu_attention(wl, si_g, lens_g)
    torch.cuda.synchronize()
    assert torch.equal(out_nolse.view(torch.int16), out_lse.view(torch.int16))
    log(f"[ok] {cfg.name}: output without lse identical to the checked one")
    free(wl)


def test_attention_at_the_split_cap():
    # one request and one 64-head group: as many column splits as compute units (256 on
    # MI355X), each of ~4 tiles, merged by the combine kernel (its LDS stage holds 256)
    cfg = WL.with_overrides(WL.CONFIGS["dense_1m"], name="dense_128k_r4_h64", ratio=4, heads=64,
                            groups=((1, 1, 1 << 17, 0),), kv_pool_pages=0)
    wl = _wl(cfg)
    c = wl.cfg
    width = c.window + wl.padded_topk
    need = sad.sparse_mla_decode_workspace_size(wl.num_tokens, c.heads, width, c.dqk)
    splits = need // (wl.num_tokens * c.heads * (c.dqk + 1) * 4)
    log(f"[report] {width} columns in {splits} splits")
    assert splits == min(torch.cuda.get_device_properties(0).multi_processor_count, (width + 31) // 32 // 4, 256)
    view = WL.host_view(wl)
    _full_check(wl, view, list(range(wl.num_tokens)))
    free(wl)


@pytest.mark.slow
def test_dense_1m_full():
    wl = _wl("dense_1m")
    view = WL.host_view(wl)
    _full_check(wl, view, list(range(wl.num_tokens)))
    free(wl)


@pytest.mark.parametrize("name", ["edge_holes", "long_ctx"])
def test_fused_indexer_and_index_build_equal_the_two_calls(name):
    # indexer_topk_sparse_indices is defined as indexer_score_topk then build_sparse_indices:
    # all three outputs bit-identical to the two-call path (with holes in both block tables
    # and a page past the pool in the "edge_holes" case).
    cfg = EDGE if name.startswith("edge") else LONG
    wl = _wl(cfg)
    L0 = wl.layers[0]
    if name == "edge_holes":
        _punch(L0.swa_bt, 0.2, 7, wl.swa_pool.shape[0] + 3)
        _punch(L0.comp_bt, 0.2, 8, wl.kv_pool.shape[0] + 3)
    tk_a, _ = gpu_indexer(wl, logits=False)
    si_a, lens_a = gpu_build(wl, tk_a)
    tk_b, si_b, lens_b = gpu_fused(wl)
    torch.cuda.synchronize()
    assert torch.equal(tk_a, tk_b)
    assert torch.equal(si_a, si_b)
    assert torch.equal(lens_a, lens_b)
    free(wl)
