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


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def caches(wl: WL.Workload):
    cfg = wl.cfg
    kv = sad.KvCache(wl.kv_pool, cfg.block, cfg.d_nope, cfg.d_rope, WL.kv_scale_format(cfg))
    idx = sad.IndexerCache(wl.idx_pool, cfg.idx_block, cfg.idx_dim)
    return kv, idx


def gpu_indexer(wl: WL.Workload, layer: int = 0, logits: bool = True):
    L = wl.layers[layer]
    _, idx = caches(wl)
    dbg = None
    if logits:
        rows = L.idx_bt.shape[1] * wl.cfg.idx_block
        dbg = torch.full((wl.num_tokens, rows), float("nan"), dtype=torch.float32, device=wl.device)
    topk = sad.indexer_score_topk(wl.query_start_loc, wl.seq_lens, wl.token_to_req, L.idx_q_values,
                                  L.idx_q_scales, L.idx_weights, idx, L.idx_bt, wl.cfg.ratio,
                                  wl.cfg.topk, logits_debug=dbg)
    return topk, dbg


def gpu_build(wl: WL.Workload, topk_local, layer: int = 0):
    L = wl.layers[layer]
    cfg = wl.cfg
    n_pages = wl.kv_pool.shape[0]
    return sad.build_sparse_indices(wl.query_start_loc, wl.seq_lens, wl.token_to_req, wl.replay_start,
                                    L.swa_bt, cfg.block, n_pages, L.comp_bt, cfg.block, n_pages,
                                    topk_local, cfg.topk, cfg.window, cfg.ratio, wl.padded_topk)


def gpu_attention(wl: WL.Workload, si, lens, layer: int = 0, sink=None, with_lse=False, q=None):
    L = wl.layers[layer]
    kv, _ = caches(wl)
    q = L.q if q is None else q
    lse = torch.empty((wl.num_tokens, wl.cfg.heads), dtype=torch.float32, device=wl.device) if with_lse else None
    out = sad.sparse_mla_decode(q, kv, kv, si, lens, wl.cfg.window, wl.padded_topk,
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
    n_pages = wl.kv_pool.shape[0]
    return O.build_sparse_indices(view.query_start_loc, view.seq_lens, view.token_to_req,
                                  view.replay_start, view.swa_bt, cfg.block, n_pages, view.comp_bt,
                                  cfg.block, n_pages, topk_local, cfg.topk, cfg.window, cfg.ratio,
                                  wl.padded_topk, tokens=tokens)


def oracle_attention(wl: WL.Workload, view, si, lens, tokens, sink=None, q_bits=None, return_mass=False):
    cfg = wl.cfg
    q_bits = view.q if q_bits is None else q_bits
    return O.sparse_mla_decode(q_bits, view.kv_pages, view.kv_pages, si, lens, cfg.window, cfg.block,
                               cfg.block, cfg.d_nope, cfg.d_rope, wl.softmax_scale, attn_sink=sink,
                               tokens=tokens, return_mass=return_mass, scale_format=cfg.kv_format)


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


def sample_tokens(wl: WL.Workload, n_decode: int, n_prefill: int, seed: int = 0):
    """Sampled tokens for oracle checks: decode tokens first, then prefill tokens
    including every prefill request's first and last token (p = 0 when its
    prefix is empty) and tokens whose window is clipped by replay_start."""
    qsl = wl.query_start_loc.cpu().numpy()
    seq = wl.seq_lens.cpu().numpy()
    rep = wl.replay_start.cpu().numpy()
    rng = np.random.default_rng(seed)
    qlen = np.diff(qsl)
    decode = [int(qsl[r]) for r in range(len(qlen)) if qlen[r] == 1]
    out = decode[:n_decode] if len(decode) <= n_decode else sorted(rng.choice(decode, n_decode, replace=False).tolist())
    pre = [r for r in range(len(qlen)) if qlen[r] > 1]
    extra = []
    for r in pre:
        first, last = int(qsl[r]), int(qsl[r + 1]) - 1
        extra += [first, last]
        p0 = seq[r] - qlen[r]
        # a token whose window reaches below replay_start
        clip = first + max(0, int(rep[r]) - int(p0))
        if first <= clip <= last:
            extra.append(clip)
        if first + 5 <= last:
            extra.append(first + 5)  # n_c < k early in a short prefix
    if pre and n_prefill:
        allp = np.concatenate([np.arange(qsl[r], qsl[r + 1]) for r in pre])
        extra += rng.choice(allp, min(n_prefill, allp.size), replace=False).tolist()
    return sorted(set(out + [int(x) for x in extra]))


def free(wl) -> None:
    del wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
