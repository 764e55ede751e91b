"""Shared plumbing for the GPU parity tests: run each step of the HIP path through
the C ABI on a seeded workload, and the matching oracle step on host copies of the
same input bytes."""

from __future__ import annotations

import sys

import numpy as np
import torch

import sparse_attention_decode_build_amd as sad
from oracle import sad_oracle as O
from sparse_attention_decode_build_amd import workloads as WL

ATOL_OUT = 5e-3
ATOL_LSE = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def kv_caches(wl: WL.Workload):
    """(window cache, compressed cache): one pool unless the config keeps two."""
    cfg = wl.cfg
    fmt = WL.kv_scale_format(cfg)
    comp = sad.KvCache(wl.kv_pool, cfg.block, cfg.d_nope, cfg.d_rope, fmt)
    swa = sad.KvCache(wl.swa_pool, cfg.swa_block_size, cfg.d_nope, cfg.d_rope, fmt)
    return swa, comp


def idx_cache(wl: WL.Workload):
    cfg = wl.cfg
    return sad.IndexerCache(wl.idx_pool, cfg.idx_block, cfg.idx_dim)


def gpu_indexer(wl: WL.Workload, layer: int = 0, logits: bool = True):
    L = wl.layers[layer]
    dbg = None
    if logits:
        rows = L.idx_bt.shape[1] * wl.cfg.idx_block
        dbg = torch.full((wl.num_tokens, rows), float("nan"), dtype=torch.float32, device=wl.device)
    topk = sad.indexer_score_topk(wl.query_start_loc, wl.seq_lens, wl.token_to_req, L.idx_q_values,
                                  L.idx_q_scales, L.idx_weights, idx_cache(wl), L.idx_bt, wl.cfg.ratio,
                                  wl.cfg.topk, logits_debug=dbg)
    return topk, dbg


def gpu_build(wl: WL.Workload, topk_local, layer: int = 0):
    L = wl.layers[layer]
    cfg = wl.cfg
    return sad.build_sparse_indices(wl.query_start_loc, wl.seq_lens, wl.token_to_req, wl.replay_start,
                                    L.swa_bt, cfg.swa_block_size, wl.swa_pool.shape[0], L.comp_bt, cfg.block,
                                    wl.kv_pool.shape[0], topk_local, cfg.topk, cfg.window, cfg.ratio,
                                    wl.padded_topk)


def gpu_fused(wl: WL.Workload, layer: int = 0):
    """indexer_topk_sparse_indices -> (topk_local, sparse_indices, lens)."""
    L = wl.layers[layer]
    c = wl.cfg
    return sad.indexer_topk_sparse_indices(
        wl.query_start_loc, wl.seq_lens, wl.token_to_req, L.idx_q_values, L.idx_q_scales, L.idx_weights,
        idx_cache(wl), L.idx_bt, c.ratio, c.topk, wl.replay_start, L.swa_bt, c.swa_block_size,
        wl.swa_pool.shape[0], L.comp_bt, c.block, wl.kv_pool.shape[0], c.window, wl.padded_topk)


def gpu_attention(wl: WL.Workload, si, lens, layer: int = 0, sink=None, with_lse=False, q=None):
    L = wl.layers[layer]
    swa, comp = kv_caches(wl)
    q = L.q if q is None else q
    lse = torch.empty((wl.num_tokens, wl.cfg.heads), dtype=torch.float32, device=wl.device) if with_lse else None
    out = sad.sparse_mla_decode(q, swa, comp, si, lens, wl.cfg.window, wl.padded_topk,
                                wl.softmax_scale, attn_sink=sink, lse=lse)
    return out, lse


def oracle_topk(wl: WL.Workload, view, tokens):
    cfg = wl.cfg
    return O.indexer_topk(view.query_start_loc, view.seq_lens, view.token_to_req, view.idx_q_values,
                          view.idx_q_scales, view.idx_weights, view.idx_pages, view.idx_bt,
                          cfg.idx_block, cfg.idx_dim, wl.idx_pool.shape[0], cfg.ratio, cfg.topk,
                          tokens=tokens, return_scores=True)


def oracle_build(wl: WL.Workload, view, topk_local, tokens=None):
    cfg = wl.cfg
    return O.build_sparse_indices(view.query_start_loc, view.seq_lens, view.token_to_req,
                                  view.replay_start, view.swa_bt, cfg.swa_block_size, wl.swa_pool.shape[0],
                                  view.comp_bt, cfg.block, wl.kv_pool.shape[0], topk_local, cfg.topk,
                                  cfg.window, cfg.ratio, wl.padded_topk, tokens=tokens)


def oracle_attention(wl: WL.Workload, view, si, lens, tokens, sink=None, q_bits=None):
    cfg = wl.cfg
    q_bits = view.q if q_bits is None else q_bits
    return O.sparse_mla_decode(q_bits, view.swa_pages, view.kv_pages, si, lens, cfg.window,
                               cfg.swa_block_size, cfg.block, cfg.d_nope, cfg.d_rope, wl.softmax_scale,
                               attn_sink=sink, tokens=tokens, scale_format=cfg.kv_format)


def oracle_gather(wl: WL.Workload, view, si, lens):
    cfg = wl.cfg
    return O.gather_dequant(view.swa_pages, view.kv_pages, si, lens, cfg.window, cfg.swa_block_size,
                            cfg.block, cfg.d_nope, cfg.d_rope, cfg.kv_format)


def check_topk(gpu_row: np.ndarray, scores: np.ndarray, valid: np.ndarray, k: int, rel: float = 1e-5):
    """GPU top-k row vs the oracle: same size, ascending valid ids, -1 padded, and the
    same set except swaps among scores within `rel` of the oracle's k-th score."""
    want = O.topk_select(scores, valid, k)
    m = int((want >= 0).sum())
    got = gpu_row[:m]
    assert np.all(gpu_row[m:] == -1), "padding must be -1"
    assert np.all(got >= 0) and np.all(np.diff(got) > 0), "ids must be valid and ascending"
    assert np.all(valid[got]), "ids must be valid rows"
    diff = set(got.tolist()) ^ set(want[:m].tolist())
    if diff:
        ids = np.nonzero(valid)[0]
        order = np.lexsort((ids, -scores[ids]))
        kth = scores[ids[order[min(k, ids.size) - 1]]]
        for x in diff:
            assert abs(scores[x] - kth) <= rel * abs(kth), (x, scores[x], kth)
    return len(diff)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def bf16_half_ulp(x):
    """Half the spacing of bfloat16 numbers at |x| (8 significant bits): the largest error
    of rounding a real number of that binade to bf16."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def check_attention(wl: WL.Workload, view, tokens, got, o_ref, si, lens, sink=None, q_bits=None,
                    label: str = "", window=None):
    """Attention output of `tokens` (got: float64 [n, H, D] of the GPU's bf16 output) vs the
    oracle's float64 o_ref.

    Bar per element: max(5e-3, half an ulp of the bf16 output + 2^-8 (1 + 2^-6) * spread
    + 2^-11 (|o| + spread)), with spread = sum_j p_j |x_j - o| (oracle.attention_spread):
    the kernel rounds every softmax weight to bf16 once (the PV MFMA's operand) and the
    output once, and accumulates in fp32.  Elements within max(5e-3, half an ulp) need no
    spread; the spread is computed only for the others.  Reports the worst error, the
    number of elements above 5e-3 and above the plain bar.  Returns the worst ratio of
    error to the plain bar max(5e-3, half an ulp)."""
    cfg = wl.cfg
    err = np.abs(got - o_ref)
    half = bf16_half_ulp(np.maximum(np.abs(o_ref), np.abs(got)))
    bar0 = np.maximum(ATOL_OUT, half)
    over = np.argwhere(err > bar0)
    n_strict = int((err > ATOL_OUT).sum())
    worst = float((err / bar0).max()) if err.size else 0.0
    if over.size:
        q_bits = view.q if q_bits is None else q_bits
        for i in np.unique(over[:, 0]):
            t = tokens[i]
            sel = over[over[:, 0] == i]
            rows = O.attended_rows(view.swa_pages, view.kv_pages, si[t], lens[t],
                                   cfg.window if window is None else window,
                                   cfg.swa_block_size, cfg.block, cfg.d_nope, cfg.d_rope, cfg.kv_format)
            sp = O.attention_spread(q_bits[t], rows, wl.softmax_scale, sink, sel[:, 1], sel[:, 2])
            for (_, h, d), s in zip(sel, sp):
                o = abs(o_ref[i, h, d])
                bar = max(ATOL_OUT, half[i, h, d] + 2.0 ** -8 * (1 + 2.0 ** -6) * s + 2.0 ** -11 * (o + s))
                assert err[i, h, d] <= bar, (f"{label} token {t} head {h} dim {d}: |err| {err[i, h, d]:.3e} > "
                                             f"{bar:.3e} (o {o_ref[i, h, d]:.4f}, spread {s:.3e})")
    rms = float(np.sqrt(np.mean((got - o_ref) ** 2)) / max(np.sqrt(np.mean(o_ref ** 2)), 1e-30))
    log(f"[report] {label} attention max-abs {err.max(initial=0.0):.3e} rel-rms {rms:.3e} "
        f"max|o| {np.abs(o_ref).max(initial=0.0):.3f}; elements > 5e-3: {n_strict} of {err.size}; "
        f"> max(5e-3, half ulp): {len(over)} (within the weight-rounding bound)")
    return worst


def sample_tokens(wl: WL.Workload, n_decode: int, n_prefill: int, seed: int = 0):
    """Sampled tokens for oracle checks: up to n_decode decode tokens, then prefill
    tokens: a seeded sample of n_prefill, every prefill request's first and last token
    (p = 0 when its prefix is empty), and of the tokens whose window is clipped by
    replay_start and of those with fewer than k compressed rows, the first, the last,
    the first past each of these ranges and 8 seeded others."""
    qsl = wl.query_start_loc.cpu().numpy()
    seq = wl.seq_lens.cpu().numpy()
    rep = wl.replay_start.cpu().numpy()
    rng = np.random.default_rng(seed)
    qlen = np.diff(qsl)
    decode = [int(qsl[r]) for r in range(len(qlen)) if qlen[r] == 1]
    out = decode if len(decode) <= n_decode else sorted(rng.choice(decode, n_decode, replace=False).tolist())
    pre = [r for r in range(len(qlen)) if qlen[r] > 1]
    extra = []
    k, W, ratio = wl.cfg.topk, wl.cfg.window, wl.cfg.ratio
    for r in pre:
        first, last = int(qsl[r]), int(qsl[r + 1]) - 1
        extra += [first, last]
        p0 = int(seq[r] - qlen[r])
        toks = np.arange(first, last + 1)
        pos = p0 + (toks - first)
        for sel in (pos - W + 1 < int(rep[r]), (pos + 1) // ratio < k if k else np.zeros_like(pos, bool)):
            ids = toks[sel]
            if ids.size:
                extra += [int(ids[0]), int(ids[-1]), min(int(ids[-1]) + 1, last)]
                extra += rng.choice(ids, min(8, ids.size), replace=False).tolist()
    if pre and n_prefill:
        allp = np.concatenate([np.arange(qsl[r], qsl[r + 1]) for r in pre])
        extra += rng.choice(allp, min(n_prefill, allp.size), replace=False).tolist()
    return sorted(set(out + [int(x) for x in extra]))


def free(wl) -> None:
    del wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
