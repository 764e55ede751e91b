"""ctypes binding of libsad.so (argument marshalling only).

Every function here takes torch device tensors, checks shapes/dtypes, passes raw
pointers plus the current HIP stream to the C ABI declared in include/sad.h and
raises on a non-OK return.  All computation happens in the HIP kernels; there is no
fallback: if libsad.so is missing or fails to load, every entry point raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsad.so")

SAD_OK, SAD_EINVAL, SAD_EUNSUPPORTED, SAD_EWORKSPACE, SAD_ELAUNCH = range(5)
_ERR = {1: "EINVAL", 2: "EUNSUPPORTED", 3: "EWORKSPACE", 4: "ELAUNCH"}

c_i32, c_i64, c_ptr, c_size, c_f32 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_float)


KV_SCALE_F32, KV_SCALE_UE8M0 = 0, 1


class SadKvCache(ctypes.Structure):
    _fields_ = [("pool", c_ptr), ("page_stride", c_i64), ("num_pages", c_i64),
                ("block_size", c_i32), ("d_nope", c_i32), ("d_rope", c_i32), ("scale_format", c_i32)]


class SadMxfp4Cache(ctypes.Structure):
    _fields_ = [("pool", c_ptr), ("page_stride", c_i64), ("num_pages", c_i64),
                ("block_size", c_i32), ("dim", c_i32)]


class SadBatch(ctypes.Structure):
    _fields_ = [("query_start_loc", c_ptr), ("seq_lens", c_ptr), ("token_to_req", c_ptr),
                ("num_reqs", c_i32), ("num_tokens", c_i32)]


_SIGNATURES = {
    "build_sparse_indices": (c_i32, [ctypes.POINTER(SadBatch), c_ptr, c_ptr, c_i64, c_i32, c_i32, c_i64,
                                     c_ptr, c_i64, c_i32, c_i32, c_i64, c_ptr, c_i64, c_i32, c_i32,
                                     c_i32, c_i32, c_ptr, c_ptr, c_ptr]),
    "indexer_score_topk": (c_i32, [ctypes.POINTER(SadBatch), c_ptr, c_ptr, c_ptr, c_i32,
                                   ctypes.POINTER(SadMxfp4Cache), c_ptr, c_i64, c_i32, c_i32, c_i32,
                                   c_ptr, c_ptr, c_i64, c_ptr, c_size, c_ptr]),
    "indexer_score_topk_workspace_size": (c_size, [c_i32, c_i32, c_i32]),
    "indexer_topk_sparse_indices": (c_i32, [ctypes.POINTER(SadBatch), c_ptr, c_ptr, c_ptr, c_i32,
                                            ctypes.POINTER(SadMxfp4Cache), c_ptr, c_i64, c_i32, c_i32, c_i32,
                                            c_ptr, c_ptr, c_ptr, c_i64, c_i32, c_i32, c_i64, c_ptr, c_i64, c_i32,
                                            c_i32, c_i64, c_i32, c_i32, c_ptr, c_ptr, c_ptr, c_size, c_ptr]),
    "prepare_indexer_q_mxfp4": (c_i32, [c_ptr, c_ptr, c_ptr, c_i32, c_i32, c_ptr, c_f32, c_f32, c_i32,
                                        c_i32, c_i32, c_ptr, c_ptr, c_ptr, c_ptr]),
    "gather_dequant_kv": (c_i32, [ctypes.POINTER(SadKvCache), ctypes.POINTER(SadKvCache), c_ptr, c_ptr,
                                  c_i32, c_i32, c_i32, c_ptr, c_ptr]),
    "sparse_mla_decode": (c_i32, [c_ptr, c_i32, c_i32, ctypes.POINTER(SadKvCache),
                                  ctypes.POINTER(SadKvCache), c_ptr, c_ptr, c_i32, c_i32, c_f32, c_ptr,
                                  c_ptr, c_ptr, c_ptr, c_size, c_ptr]),
    "sparse_mla_decode_workspace_size": (c_size, [c_i32, c_i32, c_i32, c_i32]),
    "sparse_mla_decode_noalloc": (c_i32, [c_ptr, c_i32, c_i32, ctypes.POINTER(SadKvCache),
                                          ctypes.POINTER(SadKvCache), c_ptr, c_ptr, c_i32, c_i32, c_f32, c_ptr,
                                          c_ptr, c_ptr, c_ptr]),
    "inv_rope_fp8_quant": (c_i32, [c_ptr, c_ptr, c_ptr, c_i32, c_i32, c_i32, c_i32, c_i32, c_i32, c_ptr,
                                   c_ptr, c_ptr]),
    "insert_kv_rows": (c_i32, [c_ptr, c_ptr, c_ptr, c_i32, c_i32, c_ptr, c_i32, ctypes.POINTER(SadKvCache),
                               c_ptr]),
    "insert_index_keys": (c_i32, [c_ptr, c_ptr, c_ptr, c_i32, c_i32, c_i32, c_ptr, c_i32,
                                  ctypes.POINTER(SadMxfp4Cache), c_ptr]),
    "sad_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsad.so (once) and declare the C signatures; raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it first (python -m sparse_attention_decode_build_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def last_error() -> str:
    return load().sad_last_error().decode()


def _check(name: str, rc: int) -> None:
    if rc != SAD_OK:
        raise RuntimeError(f"{name} failed with SAD_{_ERR.get(rc, rc)}: {last_error()}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, name, dim=None, device=None):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must be {dim}-D, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


@dataclass
class KvCache:
    """A paged FP8 latent cache: uint8 pool [pages, page_bytes] + its geometry and scale
    form (KV_SCALE_F32, or KV_SCALE_UE8M0 for the pages' native 448 + 64 record)."""

    pool: torch.Tensor
    block_size: int
    d_nope: int
    d_rope: int
    scale_format: int = KV_SCALE_F32

    def c(self) -> SadKvCache:
        _need(self.pool, torch.uint8, "kv pool", dim=2)
        return SadKvCache(self.pool.data_ptr(), self.pool.stride(0), self.pool.shape[0],
                          self.block_size, self.d_nope, self.d_rope, self.scale_format)


@dataclass
class IndexerCache:
    """A paged MXFP4 indexer-key cache: uint8 pool [pages, page_bytes] + geometry."""

    pool: torch.Tensor
    block_size: int
    dim: int

    def c(self) -> SadMxfp4Cache:
        _need(self.pool, torch.uint8, "indexer pool", dim=2)
        return SadMxfp4Cache(self.pool.data_ptr(), self.pool.stride(0), self.pool.shape[0],
                             self.block_size, self.dim)


def _batch(query_start_loc, seq_lens, token_to_req) -> SadBatch:
    for t, nm in ((query_start_loc, "query_start_loc"), (seq_lens, "seq_lens"),
                  (token_to_req, "token_to_req")):
        _need(t, torch.int32, nm, dim=1)
    if query_start_loc.numel() != seq_lens.numel() + 1:
        raise ValueError("query_start_loc must have num_reqs + 1 entries")
    return SadBatch(query_start_loc.data_ptr(), seq_lens.data_ptr(), token_to_req.data_ptr(),
                    seq_lens.numel(), token_to_req.numel())


def build_sparse_indices(query_start_loc, seq_lens, token_to_req, replay_start, swa_bt, swa_block_size,
                         swa_num_pages, comp_bt, comp_block_size, comp_num_pages, topk_local, topk,
                         window_size, compress_ratio, padded_topk, out=None, lens=None, stream=None):
    """Window + compressed slot ids per token -> (sparse_indices [T, W+P], lens [T])."""
    lib = load()
    b = _batch(query_start_loc, seq_lens, token_to_req)
    T = b.num_tokens
    dev = token_to_req.device
    for t, nm in ((swa_bt, "swa_bt"), (comp_bt, "comp_bt")):
        _need(t, torch.int32, nm, dim=2)
    if replay_start is not None:
        _need(replay_start, torch.int32, "replay_start", dim=1)
    if topk_local is not None:
        _need(topk_local, torch.int32, "topk_local", dim=2)
    if out is None:
        out = torch.empty((T, window_size + padded_topk), dtype=torch.int32, device=dev)
    if lens is None:
        lens = torch.empty((T,), dtype=torch.int32, device=dev)
    rc = lib.build_sparse_indices(
        ctypes.byref(b), _p(replay_start), _p(swa_bt), swa_bt.stride(0), swa_bt.shape[1],
        swa_block_size, swa_num_pages, _p(comp_bt), comp_bt.stride(0), comp_bt.shape[1],
        comp_block_size, comp_num_pages, _p(topk_local),
        topk_local.stride(0) if topk_local is not None else 0, topk, window_size, compress_ratio,
        padded_topk, _p(out), _p(lens), _stream(stream))
    _check("build_sparse_indices", rc)
    return out, lens


def indexer_topk_sparse_indices(query_start_loc, seq_lens, token_to_req, q_values, q_scales, weights,
                                keys: IndexerCache, idx_bt, compress_ratio, topk, replay_start, swa_bt,
                                swa_block_size, swa_num_pages, comp_bt, comp_block_size, comp_num_pages,
                                window_size, padded_topk, topk_local=None, out=None, lens=None,
                                workspace=None, stream=None):
    """indexer_score_topk then build_sparse_indices in one call -> (topk_local, sparse_indices, lens)."""
    lib = load()
    b = _batch(query_start_loc, seq_lens, token_to_req)
    T = b.num_tokens
    _need(q_values, torch.uint8, "q_values", dim=3)
    _need(q_scales, torch.uint8, "q_scales", dim=3)
    _need(weights, torch.float32, "weights", dim=2)
    for t, nm in ((idx_bt, "idx_bt"), (swa_bt, "swa_bt"), (comp_bt, "comp_bt")):
        _need(t, torch.int32, nm, dim=2)
    if replay_start is not None:
        _need(replay_start, torch.int32, "replay_start", dim=1)
    dev = q_values.device
    if topk_local is None:
        topk_local = torch.empty((T, topk), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty((T, window_size + padded_topk), dtype=torch.int32, device=dev)
    if lens is None:
        lens = torch.empty((T,), dtype=torch.int32, device=dev)
    max_rows = idx_bt.shape[1] * keys.block_size
    if workspace is None:
        ws = lib.indexer_score_topk_workspace_size(T, max_rows, topk)
        workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev)
    kc = keys.c()
    rc = lib.indexer_topk_sparse_indices(
        ctypes.byref(b), _p(q_values), _p(q_scales), _p(weights), q_values.shape[1], ctypes.byref(kc),
        _p(idx_bt), idx_bt.stride(0), idx_bt.shape[1], compress_ratio, topk, _p(topk_local), _p(replay_start),
        _p(swa_bt), swa_bt.stride(0), swa_bt.shape[1], swa_block_size, swa_num_pages, _p(comp_bt),
        comp_bt.stride(0), comp_bt.shape[1], comp_block_size, comp_num_pages, window_size, padded_topk,
        _p(out), _p(lens), _p(workspace), workspace.numel(), _stream(stream))
    _check("indexer_topk_sparse_indices", rc)
    return topk_local, out, lens


def prepare_indexer_q_mxfp4(index_q, positions, cos_sin_cache, weights, softmax_scale, head_scale,
                            q_values=None, q_scales=None, weights_out=None, stream=None):
    """bf16 indexer query [T, Hi, Di] -> (q_values [T, Hi, Di/2] u8, q_scales [T, Hi, Di/32] u8,
    weights_out [T, Hi] f32): RoPE tail, Hadamard rotation, MXFP4, weight fold."""
    lib = load()
    _need(index_q, torch.bfloat16, "index_q", dim=3)
    _need(positions, torch.int32, "positions", dim=1)
    _need(cos_sin_cache, torch.float32, "cos_sin_cache", dim=2)
    _need(weights, torch.float32, "weights", dim=2)
    T, H, D = index_q.shape
    if positions.shape[0] != T or tuple(weights.shape) != (T, H):
        raise ValueError("positions must be [T] and weights [T, Hi]")
    dev = index_q.device
    if q_values is None:
        q_values = torch.empty((T, H, D // 2), dtype=torch.uint8, device=dev)
    if q_scales is None:
        q_scales = torch.empty((T, H, D // 32), dtype=torch.uint8, device=dev)
    if weights_out is None:
        weights_out = torch.empty((T, H), dtype=torch.float32, device=dev)
    _need(q_values, torch.uint8, "q_values", dim=3)
    _need(q_scales, torch.uint8, "q_scales", dim=3)
    _need(weights_out, torch.float32, "weights_out", dim=2)
    if (tuple(q_values.shape) != (T, H, D // 2) or tuple(q_scales.shape) != (T, H, D // 32)
            or tuple(weights_out.shape) != (T, H)):
        raise ValueError("output shapes must be [T, Hi, Di/2], [T, Hi, Di/32] and [T, Hi]")
    rc = lib.prepare_indexer_q_mxfp4(
        _p(index_q), _p(positions), _p(cos_sin_cache), cos_sin_cache.shape[0], cos_sin_cache.shape[1],
        _p(weights), softmax_scale, head_scale, T, H, D, _p(q_values), _p(q_scales), _p(weights_out),
        _stream(stream))
    _check("prepare_indexer_q_mxfp4", rc)
    return q_values, q_scales, weights_out


def indexer_score_topk_workspace_size(num_tokens, max_ctx_rows, topk) -> int:
    return load().indexer_score_topk_workspace_size(num_tokens, max_ctx_rows, topk)


def indexer_score_topk(query_start_loc, seq_lens, token_to_req, q_values, q_scales, weights,
                       keys: IndexerCache, idx_bt, compress_ratio, topk, out=None, logits_debug=None,
                       workspace=None, stream=None):
    """MXFP4 indexer scores + per-token top-k -> topk_local [T, topk] (ascending ids, -1 pad)."""
    lib = load()
    b = _batch(query_start_loc, seq_lens, token_to_req)
    T = b.num_tokens
    _need(q_values, torch.uint8, "q_values", dim=3)
    _need(q_scales, torch.uint8, "q_scales", dim=3)
    _need(weights, torch.float32, "weights", dim=2)
    _need(idx_bt, torch.int32, "idx_bt", dim=2)
    num_heads = q_values.shape[1]
    if out is None:
        out = torch.empty((T, topk), dtype=torch.int32, device=q_values.device)
    max_rows = idx_bt.shape[1] * keys.block_size
    if workspace is None:
        ws = lib.indexer_score_topk_workspace_size(T, max_rows, topk)
        workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=q_values.device)
    if logits_debug is not None:
        _need(logits_debug, torch.float32, "logits_debug", dim=2)
    kc = keys.c()
    rc = lib.indexer_score_topk(
        ctypes.byref(b), _p(q_values), _p(q_scales), _p(weights), num_heads, ctypes.byref(kc),
        _p(idx_bt), idx_bt.stride(0), idx_bt.shape[1], compress_ratio, topk, _p(out),
        _p(logits_debug), logits_debug.stride(0) if logits_debug is not None else 0,
        _p(workspace), workspace.numel(), _stream(stream))
    _check("indexer_score_topk", rc)
    return out


def gather_dequant_kv(swa: KvCache, comp: KvCache, sparse_indices, sparse_topk_lens, window_size,
                      padded_topk, out=None, stream=None):
    """Dequantized bf16 rows of every attended column -> [T, W+P, Dn+Dr]."""
    lib = load()
    _need(sparse_indices, torch.int32, "sparse_indices", dim=2)
    _need(sparse_topk_lens, torch.int32, "sparse_topk_lens", dim=1)
    T = sparse_indices.shape[0]
    if sparse_indices.shape[1] != window_size + padded_topk:
        raise ValueError("sparse_indices must be [T, window_size + padded_topk]")
    if out is None:
        out = torch.empty((T, window_size + padded_topk, swa.d_nope + swa.d_rope), dtype=torch.bfloat16,
                          device=sparse_indices.device)
    s, c = swa.c(), comp.c()
    rc = lib.gather_dequant_kv(ctypes.byref(s), ctypes.byref(c), _p(sparse_indices),
                               _p(sparse_topk_lens), T, window_size, padded_topk, _p(out),
                               _stream(stream))
    _check("gather_dequant_kv", rc)
    return out


def sparse_mla_decode_workspace_size(num_tokens, num_heads, max_row_width, dv) -> int:
    return load().sparse_mla_decode_workspace_size(num_tokens, num_heads, max_row_width, dv)


def sparse_mla_decode(q, swa: KvCache, comp: KvCache, sparse_indices, sparse_topk_lens, window_size,
                      padded_topk, softmax_scale, attn_sink=None, out=None, lse=None, workspace=None,
                      stream=None):
    """Sparse MLA attention of every head -> out [T, H, Dn+Dr] bf16 (and lse [T, H] if given)."""
    lib = load()
    _need(q, torch.bfloat16, "q", dim=3)
    _need(sparse_indices, torch.int32, "sparse_indices", dim=2)
    _need(sparse_topk_lens, torch.int32, "sparse_topk_lens", dim=1)
    T, H, D = q.shape
    if tuple(sparse_indices.shape) != (T, window_size + padded_topk) or tuple(sparse_topk_lens.shape) != (T,):
        raise ValueError("sparse_mla_decode: sparse_indices must be [T, window_size + padded_topk] and "
                         "sparse_topk_lens [T]")
    if attn_sink is not None:
        _need(attn_sink, torch.float32, "attn_sink", dim=1)
    if out is None:
        out = torch.empty((T, H, D), dtype=torch.bfloat16, device=q.device)
    if lse is not None:
        _need(lse, torch.float32, "lse", dim=2)
    if workspace is None:
        ws = lib.sparse_mla_decode_workspace_size(T, H, window_size + padded_topk, D)
        workspace = torch.empty((max(ws, 16),), dtype=torch.uint8, device=q.device) if ws else None
    s, c = swa.c(), comp.c()
    rc = lib.sparse_mla_decode(_p(q), T, H, ctypes.byref(s), ctypes.byref(c), _p(sparse_indices),
                               _p(sparse_topk_lens), window_size, padded_topk, softmax_scale,
                               _p(attn_sink), _p(out), _p(lse), _p(workspace),
                               workspace.numel() if workspace is not None else 0, _stream(stream))
    _check("sparse_mla_decode", rc)
    return out


def sparse_mla_decode_noalloc(q, swa: KvCache, comp: KvCache, sparse_indices, sparse_topk_lens, window_size,
                              padded_topk, softmax_scale, attn_sink=None, out=None, lse=None, stream=None):
    """sparse_mla_decode without a workspace: the split partials use the library's static
    per-GPU scratch (no allocation by the library; `out` is allocated here if not given)."""
    lib = load()
    _need(q, torch.bfloat16, "q", dim=3)
    _need(sparse_indices, torch.int32, "sparse_indices", dim=2)
    _need(sparse_topk_lens, torch.int32, "sparse_topk_lens", dim=1)
    T, H, D = q.shape
    if tuple(sparse_indices.shape) != (T, window_size + padded_topk) or tuple(sparse_topk_lens.shape) != (T,):
        raise ValueError("sparse_mla_decode_noalloc: sparse_indices must be [T, window_size + padded_topk] and "
                         "sparse_topk_lens [T]")
    if attn_sink is not None:
        _need(attn_sink, torch.float32, "attn_sink", dim=1)
    if out is None:
        out = torch.empty((T, H, D), dtype=torch.bfloat16, device=q.device)
    if lse is not None:
        _need(lse, torch.float32, "lse", dim=2)
    s, c = swa.c(), comp.c()
    rc = lib.sparse_mla_decode_noalloc(_p(q), T, H, ctypes.byref(s), ctypes.byref(c), _p(sparse_indices),
                                       _p(sparse_topk_lens), window_size, padded_topk, softmax_scale,
                                       _p(attn_sink), _p(out), _p(lse), _stream(stream))
    _check("sparse_mla_decode_noalloc", rc)
    return out


def inv_rope_fp8_quant(attn_out, positions, cos_sin_cache, n_groups, out_fp8=None, out_scales=None,
                       stream=None):
    """bf16 attention output [T, H, Dh] -> (fp8 codes [G, T, D] u8, scales [G, T, D/128] f32):
    inverse RoPE of each head's tail, heads grouped, power-of-two FP8 blocks of 128."""
    lib = load()
    _need(attn_out, torch.bfloat16, "attn_out", dim=3)
    _need(positions, torch.int32, "positions", dim=1)
    _need(cos_sin_cache, torch.float32, "cos_sin_cache", dim=2)
    T, H, Dh = attn_out.shape
    if positions.shape[0] != T:
        raise ValueError("positions must be [T]")
    if n_groups < 1 or H % n_groups:
        raise ValueError("num_heads must be a multiple of n_groups")
    D = H // n_groups * Dh
    dev = attn_out.device
    if out_fp8 is None:
        out_fp8 = torch.empty((n_groups, T, D), dtype=torch.uint8, device=dev)
    if out_scales is None:
        out_scales = torch.empty((n_groups, T, max(D // 128, 1)), dtype=torch.float32, device=dev)
    _need(out_fp8, torch.uint8, "out_fp8", dim=3)
    _need(out_scales, torch.float32, "out_scales", dim=3)
    if tuple(out_fp8.shape) != (n_groups, T, D) or tuple(out_scales.shape) != (n_groups, T, D // 128):
        raise ValueError("outputs must be [G, T, D] and [G, T, D/128]")
    rc = lib.inv_rope_fp8_quant(_p(attn_out), _p(positions), _p(cos_sin_cache), cos_sin_cache.shape[0],
                                cos_sin_cache.shape[1], T, H, Dh, n_groups, _p(out_fp8), _p(out_scales),
                                _stream(stream))
    _check("inv_rope_fp8_quant", rc)
    return out_fp8, out_scales


def insert_kv_rows(rows, positions, cos_sin_cache, compress_ratio, slot_mapping, cache: KvCache, stream=None):
    """Write bf16 rows [N, Dn+Dr] (before RoPE) into the paged FP8 cache at their slots (in place)."""
    lib = load()
    _need(rows, torch.bfloat16, "rows", dim=2)
    _need(positions, torch.int32, "positions", dim=1)
    _need(cos_sin_cache, torch.float32, "cos_sin_cache", dim=2)
    _need(slot_mapping, torch.int32, "slot_mapping", dim=1)
    N = rows.shape[0]
    if positions.shape[0] != N or slot_mapping.shape[0] != N or rows.shape[1] != cache.d_nope + cache.d_rope:
        raise ValueError("rows [N, Dn+Dr], positions [N] and slot_mapping [N] must agree")
    if cos_sin_cache.shape[1] != cache.d_rope:
        raise ValueError("cos_sin_cache must be [max_pos, d_rope]")
    kc = cache.c()
    rc = lib.insert_kv_rows(_p(rows), _p(positions), _p(cos_sin_cache), cos_sin_cache.shape[0], compress_ratio,
                            _p(slot_mapping), N, ctypes.byref(kc), _stream(stream))
    _check("insert_kv_rows", rc)


def insert_index_keys(keys, positions, cos_sin_cache, compress_ratio, slot_mapping, cache: IndexerCache,
                      stream=None):
    """Write bf16 keys [N, dim] (before RoPE) into the paged MXFP4 cache at their slots (in place)."""
    lib = load()
    _need(keys, torch.bfloat16, "keys", dim=2)
    _need(positions, torch.int32, "positions", dim=1)
    _need(cos_sin_cache, torch.float32, "cos_sin_cache", dim=2)
    _need(slot_mapping, torch.int32, "slot_mapping", dim=1)
    N = keys.shape[0]
    if positions.shape[0] != N or slot_mapping.shape[0] != N or keys.shape[1] != cache.dim:
        raise ValueError("keys [N, dim], positions [N] and slot_mapping [N] must agree")
    kc = cache.c()
    rc = lib.insert_index_keys(_p(keys), _p(positions), _p(cos_sin_cache), cos_sin_cache.shape[0],
                               cos_sin_cache.shape[1], compress_ratio, _p(slot_mapping), N, ctypes.byref(kc),
                               _stream(stream))
    _check("insert_index_keys", rc)
