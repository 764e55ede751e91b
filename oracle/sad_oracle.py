"""CPU oracle for the DeepSeek-V4-style sparse-attention decode step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module:
only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
It shares no code with the HIP library (no headers, tables, helpers or
generators); it reads the same input *bytes* and recomputes every step the
plain way, in float64 where floating point is involved.

Sources (web pages; cited by page and by the function or section on it):

* [ops]     tokenspeed "DeepSeek V4 attention kernel boundaries"
            (runtime/layers/attention/deepseek_v4_ops.py page)
* [model]   tokenspeed DeepSeek V4 model page (runtime/models/deepseek_v4.py)
* [backend] tokenspeed DeepSeek V4 attention backend page
            (runtime/layers/attention/backends/deepseek_v4.py)
* [vllm]    vLLM "vllm.models.deepseek_v41.common.ops" API page

Readings taken where the pages are silent (each is listed in the design doc):

* indexer score  = sum_h w[t,h] * ReLU(q[t,h] . k_s)      (parity unpinned vs pages)
* top-k ties go to the lower row id; output is ascending by row id, -1 padded
* KV scales are fp32 per 64 nope elements (the pages use ue8m0 there); the
  pages' native ue8m0 record (448 + 64, 8 scale bytes per row) is the second form
* sparse_topk_lens counts the valid compressed entries, which are packed to
  the left of the compressed segment in top-k order; the rest is -1
* a row whose page id is negative, past the table or past the pool is invalid
  (fail closed) and is dropped
* attention values are the whole dequantized row (Dv = Dn + Dr); the sink is
  one extra logit with a zero value vector
* indexer query preparation: the RoPE output is rounded to bf16 before the
  Hadamard rotation; the rotation is a float32 radix-2 fast transform (index
  bit 0 first), times float32(D^-1/2), then bf16; the MXFP4 exponent is the smallest e with
  6 * 2^e >= amax (-127 for a zero block), codes round to nearest, ties even,
  the code's sign bit is the value's sign bit (-0.0 -> 0x8);
  weights * softmax_scale * head_scale in float32, left to right; a position
  outside the cos/sin table gives zero codes, scale byte 0 and weight 0
* output inverse RoPE + FP8: the rotated values are quantized in float32
  (no bf16 step); power-of-two scales 2^e with e the smallest integer with
  448 * 2^e >= amax, at least -33; blocks of 128 run along each group's row
  and may span two heads; output group major [G, T, D]; a position outside
  the table gives zero codes and zero scales
* cache write side: RoPE at the compressed position floor(p / ratio) * ratio;
  KV nope scales in the fp32 form, float32(max(amax, 1e-4)) / 448, codes
  e4m3(clamp(x / scale)) with float32 division; indexer keys take the query's
  RoPE -> bf16 -> rotation -> MXFP4 steps; a negative slot, a page past the pool
  or a position outside the cos/sin table is skipped
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# O2: element codecs
# ---------------------------------------------------------------------------


def e4m3fn_value(byte: int) -> float:
    """Value of one OCP FP8 E4M3 ("fn") byte.

    Sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 is
    subnormal (m/8 * 2^-6); there are no infinities and S.1111.111 is NaN, so
    the largest finite magnitude is 448.  gfx950 uses this OCP encoding, not
    the FNUZ one ([vllm] ``dequantize_and_gather_k_cache``, use_fnuz note).
    """
    sign = -1.0 if byte & 0x80 else 1.0
    exp = (byte >> 3) & 0xF
    man = byte & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


E4M3_VALUES = np.array([e4m3fn_value(b) for b in range(256)], dtype=np.float64)

# [ops] ``_e2m1_values``: magnitudes of the 3 low bits, sign in bit 3.
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_value(nibble: int) -> float:
    mag = E2M1_MAGNITUDES[nibble & 0x7]
    return -mag if nibble & 0x8 else mag


E2M1_VALUES = np.array([e2m1_value(n) for n in range(16)], dtype=np.float64)


def e8m0_value(byte: int) -> float:
    """[ops] ``read_deepseek_v4_indexer_mxfp4_cache``: scale = 2^(b - 127)."""
    return math.ldexp(1.0, int(byte) - 127)


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32; returns float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def float32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bfloat16, nearest-even; returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return out


# ---------------------------------------------------------------------------
# O1: token geometry
# ---------------------------------------------------------------------------


def token_positions(query_start_loc, seq_lens, token_to_req) -> np.ndarray:
    """Position of every token in its request.

    [backend] ``_decode_positions_from_metadata``:
    ``pos = seq_len - query_len + (t - query_start)`` for the token's request,
    where seq_len counts this step's query tokens.
    """
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    req = np.asarray(token_to_req, dtype=np.int64)
    t = np.arange(req.shape[0], dtype=np.int64)
    if req.size:
        if not np.all((qsl[req] <= t) & (t < qsl[req + 1])):
            raise ValueError("token_to_req disagrees with query_start_loc")
    qlen = qsl[req + 1] - qsl[req]
    return sl[req] - qlen + (t - qsl[req])


def compressed_len(pos: np.ndarray, ratio: int) -> np.ndarray:
    """Compressed rows visible to a token at ``pos``: floor((pos + 1) / ratio).

    A compressed row is complete once ``(pos + 1) % ratio == 0`` ([ops]
    compressor helpers; [model] indexer prefill ``row_lens``; [backend]
    dense compressed indices).
    """
    return np.maximum(np.asarray(pos, dtype=np.int64) + 1, 0) // int(ratio)


# ---------------------------------------------------------------------------
# O5/O6: slot mapping, window ids, sparse index rows
# ---------------------------------------------------------------------------


def logical_to_slot(bt_row, logical: int, block_size: int, num_pages: int) -> int:
    """Paged lookup ``bt[logical // B] * B + logical % B``, or -1 (fail closed).

    [vllm] ``compute_global_topk_indices_and_lens`` (block-table lookup),
    [backend] dense compressed indices (``safe_page_ids``; invalid -> -1).
    """
    if logical < 0:
        return -1
    col = logical // block_size
    if col >= len(bt_row):
        return -1
    page = int(bt_row[col])
    if page < 0 or page >= num_pages:
        return -1
    return page * block_size + logical % block_size


def _slots(bt_row, logical, block_size, num_pages):
    """Vector form of ``logical_to_slot`` for an array of logical rows."""
    logical = np.asarray(logical, dtype=np.int64)
    bt_row = np.asarray(bt_row, dtype=np.int64)
    col = np.where(logical >= 0, logical // block_size, 0)
    inside = (logical >= 0) & (col < bt_row.shape[0])
    page = np.where(inside, bt_row[np.minimum(col, max(bt_row.shape[0] - 1, 0))] if bt_row.size else -1, -1)
    ok = inside & (page >= 0) & (page < num_pages)
    return np.where(ok, page * block_size + logical % block_size, -1)


def build_sparse_indices(
    query_start_loc, seq_lens, token_to_req, replay_start,
    swa_bt, swa_block_size, swa_num_pages,
    comp_bt, comp_block_size, comp_num_pages,
    topk_local, topk, window_size, compress_ratio, padded_topk, tokens=None,
):
    """One int32 row per token: ``window_size`` window slots then ``padded_topk``
    compressed slots, plus the count of valid compressed slots.

    Window columns ([vllm] ``build_flashinfer_mixed_sparse_indices``; [backend]
    ``_update_decode_swa_metadata``): positions ``lo..pos`` ascending with
    ``lo = max(pos - W + 1, replay_start[r], 0)`` mapped through the window
    table, then -1.  Compressed columns ([vllm]
    ``compute_global_topk_indices_and_lens``; [backend]
    ``_decode_compressed_attention_indices_and_lens``): each local id of the
    token's top-k row (or ``0..n_c-1`` when ``topk_local`` is None, the dense
    ratio-128 path) that is ``< n_c`` and maps to a backed page, in order,
    packed left; then -1.  ``tokens`` restricts the output rows to those tokens.
    """
    pos = token_positions(query_start_loc, seq_lens, token_to_req)
    req = np.asarray(token_to_req, dtype=np.int64)
    replay = np.zeros(len(seq_lens), np.int64) if replay_start is None else np.asarray(replay_start)
    tokens = list(range(req.shape[0])) if tokens is None else list(tokens)
    W, P = int(window_size), int(padded_topk)
    out = np.full((len(tokens), W + P), -1, dtype=np.int32)
    lens = np.zeros(len(tokens), dtype=np.int32)
    nc_all = compressed_len(pos, compress_ratio)
    for i, t in enumerate(tokens):
        r = int(req[t])
        p = int(pos[t])
        lo = max(p - W + 1, int(replay[r]), 0)
        window = np.arange(lo, p + 1)
        out[i, : window.size] = _slots(swa_bt[r], window, swa_block_size, swa_num_pages)
        nc = int(nc_all[t])
        if topk_local is None:
            cand = np.arange(min(nc, P))
        else:
            cand = np.asarray(topk_local[t, :topk], dtype=np.int64)
        cand = cand[(cand >= 0) & (cand < nc)]
        slots = _slots(comp_bt[r], cand, comp_block_size, comp_num_pages)
        slots = slots[slots >= 0]
        out[i, W: W + slots.size] = slots
        lens[i] = slots.size
    return out, lens


# ---------------------------------------------------------------------------
# O7: latent row dequantization
# ---------------------------------------------------------------------------


def kv_scale_bytes(d_nope: int, scale_format: str = "f32") -> int:
    """Bytes of one row's scales: d_nope/64 fp32 (the fp32 form), or the pages' native
    ue8m0 form, one byte per 64 nope values padded to 8 bytes ([ops]
    ``deepseek_v4_swa_scale_dim``: 448 nope values -> 7 scales + 1 pad byte)."""
    return 4 * (d_nope // 64) if scale_format == "f32" else 8


def dequant_rows(kv_pages: dict, slots, block_size: int, d_nope: int, d_rope: int,
                 scale_format: str = "f32") -> np.ndarray:
    """bf16 bits [n, Dn+Dr] of the rows at ``slots``; slot -1 gives a zero row.

    [ops] ``dequantize_deepseek_v4_fp8_ds_mla_cache``: values of row ``o`` of
    page ``g`` start at ``g*stride + o*(Dn + 2*Dr)``; its scales start at
    ``g*stride + B*(Dn + 2*Dr) + o*scale_bytes``.  Each nope element is
    ``bf16_rne(fp32(e4m3(v)) * scale[d // 64])`` (one binary32 multiply); the
    rope tail is stored bf16 and copied.  Scales are fp32 (4 bytes each) in the
    "f32" form, or the pages' ue8m0 bytes, scale = 2^(b - 127), in the "ue8m0"
    form (where the product is exact).
    """
    slots = np.asarray(slots, dtype=np.int64)
    row_b = d_nope + 2 * d_rope
    nsc = d_nope // 64
    sbytes = kv_scale_bytes(d_nope, scale_format)
    out = np.zeros((slots.shape[0], d_nope + d_rope), dtype=np.uint16)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        page = kv_pages[int(s) // block_size]
        o = int(s) % block_size
        vals = page[o * row_b: (o + 1) * row_b]
        sbase = block_size * row_b + o * sbytes
        if scale_format == "f32":
            scales = page[sbase: sbase + 4 * nsc].view(np.float32)
        else:
            scales = np.ldexp(np.float32(1.0), page[sbase: sbase + nsc].astype(np.int32) - 127).astype(np.float32)
        nope32 = E4M3_VALUES[vals[:d_nope]].astype(np.float32)
        prod = nope32 * np.repeat(scales, 64)  # binary32 multiply
        out[i, :d_nope] = float32_to_bf16_bits(prod)
        out[i, d_nope:] = vals[d_nope:].view(np.uint16)
    return out


def gather_dequant(kv_swa: dict, kv_comp: dict, sparse_indices, sparse_topk_lens,
                   window_size, block_size_swa, block_size_comp, d_nope, d_rope,
                   scale_format: str = "f32") -> np.ndarray:
    """[T, W+P, Dn+Dr] bf16 bits: every attended column dequantized, others zero.

    Window columns read the window cache; compressed columns ``W..W+lens-1``
    read the compressed cache; -1 and columns past ``lens`` are zero rows.
    """
    si = np.asarray(sparse_indices)
    T, width = si.shape
    W = int(window_size)
    out = np.zeros((T, width, d_nope + d_rope), dtype=np.uint16)
    for t in range(T):
        out[t, :W] = dequant_rows(kv_swa, si[t, :W], block_size_swa, d_nope, d_rope, scale_format)
        n = int(min(max(sparse_topk_lens[t], 0), width - W))
        out[t, W: W + n] = dequant_rows(kv_comp, si[t, W: W + n], block_size_comp, d_nope, d_rope,
                                        scale_format)
    return out


# ---------------------------------------------------------------------------
# O3/O4: indexer scores and top-k
# ---------------------------------------------------------------------------


def mxfp4_decode(packed: np.ndarray, exps: np.ndarray) -> np.ndarray:
    """[n, D/2] packed E2M1 + [n, D/32] e8m0 -> float64 [n, D].

    [ops] ``read_deepseek_v4_indexer_mxfp4_cache``: the low nibble is the
    even element, the high nibble the odd one; every 32 elements share one
    power-of-two scale.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    n, half = packed.shape
    vals = np.empty((n, 2 * half), dtype=np.float64)
    vals[:, 0::2] = E2M1_VALUES[packed & 0xF]
    vals[:, 1::2] = E2M1_VALUES[packed >> 4]
    scale = np.ldexp(1.0, np.asarray(exps, dtype=np.int64) - 127)
    return vals * np.repeat(scale, 32, axis=1)


def read_index_keys(idx_pages: dict, bt_row, rows: int, block_size: int, dim: int, num_pages: int):
    """Keys of compressed rows ``0..rows-1`` through the indexer table.

    Returns (keys float64 [rows, dim], valid bool [rows]); a row whose page is
    unbacked is invalid and its key is zero.
    """
    vb, sb = dim // 2, dim // 32
    keys = np.zeros((rows, dim), dtype=np.float64)
    valid = np.zeros(rows, dtype=bool)
    for c in range((rows + block_size - 1) // block_size):
        lo, hi = c * block_size, min(rows, (c + 1) * block_size)
        if c >= len(bt_row):
            break
        page_id = int(bt_row[c])
        if page_id < 0 or page_id >= num_pages:
            continue
        page = idx_pages[page_id]
        n = hi - lo
        packed = page[: block_size * vb].reshape(block_size, vb)[:n]
        exps = page[block_size * vb: block_size * (vb + sb)].reshape(block_size, sb)[:n]
        keys[lo:hi] = mxfp4_decode(packed, exps)
        valid[lo:hi] = True
    return keys, valid


def indexer_scores(q_values, q_scales, weights, keys) -> np.ndarray:
    """score[s] = sum_h w[h] * max(q_h . k_s, 0), float64.

    Per token, each indexer head's MXFP4 query is dotted with every compressed
    row's MXFP4 key, and the per-head logits are combined with the folded
    weights ([model] ``_deepseek_v4_indexer_topk_from_cache_deepgemm_decode``;
    [vllm] ``fused_indexer_q_rope_quant``: MXFP4 weights carry
    softmax_scale * head_scale).  The ReLU combination is this build's reading.
    """
    q = mxfp4_decode(q_values, q_scales)  # [Hi, Di]
    dots = q @ keys.T  # [Hi, n]
    return np.asarray(weights, dtype=np.float64) @ np.maximum(dots, 0.0)


def topk_select(scores: np.ndarray, valid: np.ndarray, k: int) -> np.ndarray:
    """Ids of the ``min(k, #valid)`` largest scores (ties: lower id), ascending,
    -1 padded to ``k`` ([model] ``_deepseek_v4_indexer_topk_from_logits``:
    the output starts filled with -1)."""
    ids = np.nonzero(valid)[0]
    out = np.full(k, -1, dtype=np.int32)
    if ids.size == 0 or k == 0:
        return out
    order = np.lexsort((ids, -scores[ids]))
    chosen = np.sort(ids[order[:k]])
    out[: chosen.size] = chosen
    return out


def indexer_topk(query_start_loc, seq_lens, token_to_req, q_values, q_scales, weights,
                 idx_pages, idx_bt, idx_block_size, idx_dim, idx_num_pages, compress_ratio, topk,
                 tokens=None, return_scores=False):
    """Top-k local compressed-row ids for each token (all, or ``tokens``)."""
    pos = token_positions(query_start_loc, seq_lens, token_to_req)
    nc = compressed_len(pos, compress_ratio)
    req = np.asarray(token_to_req, dtype=np.int64)
    tokens = range(req.shape[0]) if tokens is None else tokens
    out = np.full((len(tokens), topk), -1, dtype=np.int32)
    scores_out = []
    # a request's keys are read once, for its widest token (rows 0..n-1 of a read of
    # more rows are the same rows)
    widest = {}
    for t in tokens:
        widest[int(req[t])] = max(widest.get(int(req[t]), 0), int(nc[t]))
    keys_of = {r: read_index_keys(idx_pages, idx_bt[r], n, idx_block_size, idx_dim, idx_num_pages)
               for r, n in widest.items()}
    for i, t in enumerate(tokens):
        n = int(nc[t])
        all_keys, all_valid = keys_of[int(req[t])]
        keys, valid = all_keys[:n], all_valid[:n]
        sc = indexer_scores(q_values[t], q_scales[t], weights[t], keys) if n else np.zeros(0)
        out[i] = topk_select(sc, valid, topk)
        scores_out.append((sc, valid))
    return (out, scores_out) if return_scores else out


# ---------------------------------------------------------------------------
# O8: attention
# ---------------------------------------------------------------------------


def attend(q_bits: np.ndarray, row_bits: np.ndarray, softmax_scale: float, sink=None,
           return_mass: bool = False):
    """Softmax attention of every head over the given rows (float64).

    ``o_h = sum_j exp(l_hj - m) x_j / (sum_j exp(l_hj - m) + exp(sink_h - m))``
    with ``l_hj = c * q_h . x_j`` over the full row, ``m`` the max of the
    logits and the sink ([backend] ``forward_deepseek_v4_decode``: values are
    the whole row, ``head_dim_v = head_dim``; [model] attention: scale
    ``head_dim^-1/2``, per-head sink).  Returns (o [H, D], lse [H]); with no
    rows and no sink, o = 0 and lse = -inf.  With ``return_mass`` also returns
    ``sum_j p_j |x_j|`` per head and dim, the scale of any per-weight rounding error.
    """
    q = bf16_bits_to_float(q_bits)  # [H, D]
    H = q.shape[0]
    if row_bits.shape[0] == 0 and sink is None:
        zero = np.zeros((H, row_bits.shape[1]), np.float64)
        return (zero, np.full(H, -np.inf), zero) if return_mass else (zero, np.full(H, -np.inf))
    x = bf16_bits_to_float(row_bits)  # [n, D]
    logits = softmax_scale * (q @ x.T)  # [H, n]
    s = None if sink is None else np.asarray(sink, dtype=np.float64)
    m = logits.max(axis=1) if logits.shape[1] else np.full(H, -np.inf)
    if s is not None:
        m = np.maximum(m, s)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(logits - m_safe[:, None])
    z = e.sum(axis=1)
    if s is not None:
        z = z + np.exp(s - m_safe)
    zs = np.where(z > 0, z, 1.0)[:, None]
    o = (e @ x) / zs
    o[z == 0] = 0.0
    with np.errstate(divide="ignore"):
        lse = m_safe + np.log(z)
    if return_mass:
        mass = (e @ np.abs(x)) / zs
        mass[z == 0] = 0.0
        return o, lse, mass
    return o, lse


def attention_spread(q_bits: np.ndarray, row_bits: np.ndarray, softmax_scale: float, sink,
                     heads, dims) -> np.ndarray:
    """``sum_j p_j |x_j[d] - o[h, d]|`` for each given (head h, dim d) pair, float64.

    ``p_j`` are the normalized softmax weights of ``attend`` (the sink included in the
    denominator) and ``o`` its output.  A relative change ``d_j`` of every weight,
    renormalized, moves ``o[h, d]`` by ``sum_j p_j d_j (x_j[d] - o[h, d])``, so one
    rounding of every weight to a format with unit roundoff u moves it by at most u
    times this sum.  Zero where nothing is attended.
    """
    heads = np.asarray(heads, dtype=np.int64)
    dims = np.asarray(dims, dtype=np.int64)
    out = np.zeros(heads.shape[0], np.float64)
    if row_bits.shape[0] == 0:
        return out
    q = bf16_bits_to_float(q_bits)
    x = bf16_bits_to_float(row_bits)
    o, _ = attend(q_bits, row_bits, softmax_scale, sink)
    for i, (h, d) in enumerate(zip(heads, dims)):
        logits = softmax_scale * (x @ q[h])
        m = logits.max()
        if sink is not None:
            m = max(m, float(sink[h]))
        e = np.exp(logits - m)
        z = e.sum() + (math.exp(float(sink[h]) - m) if sink is not None else 0.0)
        out[i] = float(e @ np.abs(x[:, d] - o[h, d])) / z
    return out


def attended_rows(kv_swa, kv_comp, si_row, topk_len, window_size, block_size_swa, block_size_comp,
                  d_nope, d_rope, scale_format="f32") -> np.ndarray:
    """bf16 bits [n, Dn+Dr] of one token's attended rows: window columns ``0..W-1`` with
    a slot >= 0 read from the window cache, then compressed columns ``W..W+lens-1`` with
    a slot >= 0 read from the compressed cache ([backend] ``forward_deepseek_v4_decode``:
    ``k_cache`` is the window cache, ``extra_k_cache`` the compressed one)."""
    si_row = np.asarray(si_row)
    W = int(window_size)
    swa = si_row[:W]
    n = int(min(max(int(topk_len), 0), si_row.shape[0] - W))
    comp = si_row[W: W + n]
    return np.concatenate([
        dequant_rows(kv_swa, swa[swa >= 0], block_size_swa, d_nope, d_rope, scale_format),
        dequant_rows(kv_comp, comp[comp >= 0], block_size_comp, d_nope, d_rope, scale_format),
    ])


def sparse_mla_decode(q_bits, kv_swa, kv_comp, sparse_indices, sparse_topk_lens, window_size,
                      block_size_swa, block_size_comp, d_nope, d_rope, softmax_scale,
                      attn_sink=None, tokens=None, return_mass=False, scale_format="f32"):
    """Attention of every head of each token over its attended columns.

    Attended columns: window columns ``0..W-1`` with slot >= 0 and compressed
    columns ``W..W+lens-1`` with slot >= 0, each one key ([backend]
    ``forward_deepseek_v4_decode``: window ids bounded by their lengths plus
    extra (compressed) ids bounded by ``extra_topk_length``).
    Returns float64 (o [n, H, Dn+Dr], lse [n, H]) and, with ``return_mass``, the
    per-output absolute mass ``sum_j p_j |x_j|`` [n, H, Dn+Dr].
    """
    si = np.asarray(sparse_indices)
    W = int(window_size)
    tokens = range(si.shape[0]) if tokens is None else tokens
    H = q_bits.shape[1]
    D = d_nope + d_rope
    o = np.zeros((len(tokens), H, D), np.float64)
    lse = np.zeros((len(tokens), H), np.float64)
    mass = np.zeros((len(tokens), H, D), np.float64) if return_mass else None
    for i, t in enumerate(tokens):
        rows = attended_rows(kv_swa, kv_comp, si[t], sparse_topk_lens[t], W, block_size_swa,
                             block_size_comp, d_nope, d_rope, scale_format)
        if return_mass:
            o[i], lse[i], mass[i] = attend(q_bits[t], rows, softmax_scale, attn_sink, return_mass=True)
        else:
            o[i], lse[i] = attend(q_bits[t], rows, softmax_scale, attn_sink)
    return (o, lse, mass) if return_mass else (o, lse)


# ---------------------------------------------------------------------------
# Indexer query preparation: RoPE tail -> Hadamard -> MXFP4, weight fold
# ---------------------------------------------------------------------------


def rope_gptj_tail(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, rope_dim: int) -> np.ndarray:
    """GPT-J (interleaved) rotary embedding of the last ``rope_dim`` elements, float32.

    [ops] rotary tail of the indexer query (GPT-J style, ``is_neox_style=False`` on the
    [model] page): element pair i of the tail, (e, o) at positions (n + 2i, n + 2i + 1)
    with n = D - rope_dim, is the complex number e + i*o, and it is multiplied by
    cos_i + i*sin_i, giving (e*cos_i - o*sin_i, e*sin_i + o*cos_i).  Every real product
    and sum of that complex multiply is a separate float32 operation (no fused
    multiply-add).  ``x`` [..., D]; ``cos``/``sin`` [..., rope_dim/2] share ``x``'s
    leading axes and broadcast over any axes between them and the last.  The leading
    part of each row is returned unchanged.
    """
    f32 = np.float32
    out = np.array(x, dtype=f32, copy=True)
    n = out.shape[-1] - rope_dim
    c = np.asarray(cos, dtype=f32)
    s = np.asarray(sin, dtype=f32)
    extra = out.ndim - c.ndim  # axes of x between cos/sin's leading axes and the last one
    lead = c.shape[:-1]
    for i in range(rope_dim // 2):
        ci = c[..., i].reshape(lead + (1,) * extra)
        si = s[..., i].reshape(lead + (1,) * extra)
        re = out[..., n + 2 * i].copy()
        im = out[..., n + 2 * i + 1].copy()
        out[..., n + 2 * i] = f32(re * ci) - f32(im * si)
        out[..., n + 2 * i + 1] = f32(re * si) + f32(im * ci)
    return out


def hadamard_matrix(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two): H[i, j] = (-1)^popcount(i & j)."""
    i = np.arange(n)
    bits = np.bitwise_and.outer(i, i)
    parity = np.zeros_like(bits)
    while bits.any():
        parity ^= bits & 1
        bits >>= 1
    return np.where(parity == 1, -1.0, 1.0)


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Fast Walsh-Hadamard transform of rows [..., D] in float32 (unscaled).

    Radix-2 stages over the element-index bits, bit 0 first: at stage s (s =
    1, 2, 4, ...) each pair (i, i + s) with bit s of i clear becomes
    (x_i + x_{i+s}, x_i - x_{i+s}), each a float32 sum.  With exact arithmetic
    this is H x for the Sylvester matrix H of ``hadamard_matrix``.
    """
    y = np.array(x, dtype=np.float32, copy=True)
    lead, d = y.shape[:-1], y.shape[-1]
    y = y.reshape(-1, d)
    s = 1
    while s < d:
        v = y.reshape(-1, d // (2 * s), 2, s)
        a = v[:, :, 0, :].copy()
        b = v[:, :, 1, :].copy()
        v[:, :, 0, :] = a + b
        v[:, :, 1, :] = a - b
        s *= 2
    return y.reshape(*lead, d)


def hadamard_rotate(x_bf16_bits: np.ndarray) -> np.ndarray:
    """Scaled Hadamard rotation of bf16 rows; returns bf16 bits.

    [ops] ``_deepseek_v4_hadamard_rotate``: the rows are bf16, the transform is
    the Sylvester Hadamard matrix with scale D^-1/2, computed in float32, and
    the result is bf16.  Reading of the float32 arithmetic: the radix-2 fast
    transform of ``fwht_f32`` (index bit 0 first), then one float32 multiply by
    float32(D^-1/2), then bf16 rounding (nearest even).
    """
    x = bf16_bits_to_float(x_bf16_bits).astype(np.float32)
    d = x.shape[-1]
    y = (fwht_f32(x) * np.float32(d ** -0.5)).astype(np.float32)
    return float32_to_bf16_bits(y)


def mxfp4_encode(x: np.ndarray):
    """Values [..., D] -> (packed E2M1 nibbles [..., D/2] u8, e8m0 bytes [..., D/32] u8).

    Per 32 consecutive elements with largest magnitude a: the shared exponent e
    is the smallest integer with 6 * 2^e >= a (6 is the largest E2M1 magnitude;
    the analogue of the pages' FP8 rule scale = amax / max), e = -127 when a is
    zero, clamped to [-127, 127]; its byte is e + 127 ([ops]
    ``read_deepseek_v4_indexer_mxfp4_cache``: scale 2^(b-127)).  Each element
    becomes the E2M1 code whose magnitude ([ops] ``_e2m1_values``) is nearest
    to |x| / 2^e, a tie going to the even code; its sign bit (0x8) is the
    sign bit of x, so -0.0 encodes as 0x8 (the IEEE reading of a sign).  The
    even element is the low nibble.
    """
    x = np.asarray(x, dtype=np.float64)
    lead, d = x.shape[:-1], x.shape[-1]
    blocks = x.reshape(-1, d // 32, 32)
    exps = np.empty(blocks.shape[:2], dtype=np.int64)
    codes = np.empty(blocks.shape, dtype=np.uint8)
    mags = np.array(E2M1_MAGNITUDES)
    for r in range(blocks.shape[0]):
        for b in range(blocks.shape[1]):
            blk = blocks[r, b]
            a = float(np.max(np.abs(blk)))
            if a == 0.0:
                e = -127
            else:
                e = math.ceil(math.log2(a / 6.0))
                while 6.0 * 2.0 ** (e - 1) >= a:
                    e -= 1
                while 6.0 * 2.0 ** e < a:
                    e += 1
                e = min(max(e, -127), 127)
            exps[r, b] = e
            for j in range(32):
                v = abs(blk[j]) / 2.0 ** e
                dist = np.abs(mags - v)
                best = int(np.flatnonzero(dist == dist.min())[0])
                if best + 1 < 8 and dist[best + 1] == dist[best] and best % 2 == 1:
                    best += 1
                codes[r, b, j] = best | (0x8 if np.signbit(blk[j]) else 0)
    codes = codes.reshape(-1, d)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return (packed.reshape(*lead, d // 2),
            (exps + 127).astype(np.uint8).reshape(*lead, d // 32))


def fold_index_weights(weights: np.ndarray, softmax_scale: float, head_scale: float) -> np.ndarray:
    """[vllm] ``fused_indexer_q_rope_quant``, MXFP4 path: weights * softmax_scale * head_scale.

    Float32, left to right (the block scales stay with the MXFP4 query).
    """
    w = np.asarray(weights, dtype=np.float32)
    return ((w * np.float32(softmax_scale)).astype(np.float32) * np.float32(head_scale)).astype(np.float32)


def prepare_indexer_q_mxfp4(index_q_bits, positions, cos_sin_cache, weights, softmax_scale, head_scale):
    """Indexer query -> the scorer's MXFP4 inputs.

    [ops] ``deepseek_v4_prepare_indexer_q_mxfp4`` (RoPE, then the Hadamard
    rotation, then MXFP4) and [vllm] ``fused_indexer_q_rope_quant`` (MXFP4
    outputs and the weight fold).  ``index_q_bits`` [T, Hi, Di] bf16 bits;
    ``positions`` [T]; ``cos_sin_cache`` [P, R] float32 (cos in the first R/2
    columns, sin in the rest); ``weights`` [T, Hi] float32.  The RoPE output is
    rounded to bf16 before the rotation, as the rotation takes bf16 rows.  A
    token whose position is outside [0, P) is failed closed: zero codes, scale
    byte 0, folded weight 0.
    Returns (q_values [T, Hi, Di/2] u8, q_scales [T, Hi, Di/32] u8, weights_out [T, Hi] f32).
    """
    q = bf16_bits_to_float(index_q_bits)
    T, H, D = q.shape
    cs = np.asarray(cos_sin_cache, dtype=np.float32)
    P, R = cs.shape
    pos = np.asarray(positions, dtype=np.int64)
    ok = (pos >= 0) & (pos < P)
    pc = np.where(ok, pos, 0)
    roped = rope_gptj_tail(q.astype(np.float32), cs[pc, : R // 2], cs[pc, R // 2:], R)
    rotated = hadamard_rotate(float32_to_bf16_bits(roped))
    values, scales = mxfp4_encode(bf16_bits_to_float(rotated))
    w_out = fold_index_weights(weights, softmax_scale, head_scale)
    values[~ok] = 0
    scales[~ok] = 0
    w_out[~ok] = 0.0
    return values, scales, w_out


# ---------------------------------------------------------------------------
# After attention: inverse RoPE on each head's tail + grouped FP8 quantization
# ---------------------------------------------------------------------------


def inv_rope_gptj_tail(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, rope_dim: int) -> np.ndarray:
    """Inverse of ``rope_gptj_tail``: each tail pair (e, o) rotated by -angle, float32.

    [ops] model page: the attention RoPE is GPT-J style (``is_neox_style=False``,
    cos/sin table with the cos half first); [vllm] ``fused_inv_rope_fp8_quant``
    undoes it on the attention output.  (e, o) -> (e*cos + o*sin, o*cos - e*sin),
    every product and sum a separate float32 operation.
    """
    out = np.array(x, dtype=np.float32, copy=True)
    n = out.shape[-1] - rope_dim
    e = out[..., n::2].copy()
    o = out[..., n + 1::2].copy()
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    while c.ndim < e.ndim:
        c = c[..., None, :]
        s = s[..., None, :]
    out[..., n::2] = (e * c).astype(np.float32) + (o * s).astype(np.float32)
    out[..., n + 1::2] = (o * c).astype(np.float32) - (e * s).astype(np.float32)
    return out


_E4M3_POS = E4M3_VALUES[:127]  # codes 0x00..0x7E: 0 .. 448, ascending


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float values with |x| <= 448 -> OCP e4m3fn bytes, nearest value, ties to the even code.

    The sign bit is copied from x (so -0.0 -> 0x80), as a float conversion does.
    """
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    codes = np.empty(flat.shape, dtype=np.uint8)
    for lo in range(0, len(flat), 1 << 16):  # in chunks, to bound the distance table
        xs = flat[lo: lo + (1 << 16)]
        dist = np.abs(np.abs(xs)[:, None] - _E4M3_POS[None, :])
        best = np.argmin(dist, axis=1)
        nxt = np.minimum(best + 1, 126)
        r = np.arange(len(best))
        tie = (dist[r, nxt] == dist[r, best]) & (nxt != best)
        best = np.where(tie & (best % 2 == 1), nxt, best)
        codes[lo: lo + len(xs)] = best.astype(np.uint8) | np.where(np.signbit(xs), 0x80, 0).astype(np.uint8)
    return codes.reshape(x.shape)


def fp8_pow2_quant(blocks: np.ndarray):
    """Blocks [..., B] -> (e4m3fn bytes [..., B], float32 scales [...]), power-of-two scales.

    [ops] ``_fp8_e4m3_pow2_bytes``: scale = 2^ceil(log2(max(amax / 448, 1e-10))),
    values = e4m3(clamp(x / scale, +-448)).  Written exactly: e is the smallest
    integer with 448 * 2^e >= amax, and at least -33 (2^-34 < 1e-10 <= 2^-33).
    """
    blocks = np.asarray(blocks, dtype=np.float64)
    amax = np.abs(blocks).max(axis=-1)
    e = np.empty(amax.shape, dtype=np.int64)
    for idx, a in np.ndenumerate(amax):
        k = -33
        if a > 0.0:
            k = math.ceil(math.log2(a / 448.0))
            while 448.0 * 2.0 ** (k - 1) >= a:
                k -= 1
            while 448.0 * 2.0 ** k < a:
                k += 1
        e[idx] = max(k, -33)
    scale = np.ldexp(1.0, e)
    y = np.clip(blocks / scale[..., None], -448.0, 448.0)
    return e4m3_encode(y), scale.astype(np.float32)


def inv_rope_fp8_quant(o_bits, positions, cos_sin_cache, n_groups: int, rope_dim: int, block: int = 128):
    """Attention output -> the output projection's grouped FP8 input.

    [vllm] ``fused_inv_rope_fp8_quant`` and [model] ``_project_attention_output``:
    ``o_bits`` [T, H, Dh] bf16 bits; each head's last ``rope_dim`` elements get
    the inverse GPT-J RoPE at ``positions[t]`` (float32); the heads are taken
    in groups of H / n_groups, and each group's row of D = (H / n_groups) * Dh
    values (heads in order, then dims) is quantized in blocks of ``block``
    consecutive values with ``fp8_pow2_quant``.  Readings: the rotated values
    go to the quantizer in float32 (no bf16 step between), blocks may span two
    heads (only D needs to be a multiple of the block), the output is group
    major as the pages' buffer is, and a token whose position is outside the
    table is failed closed (zero codes, zero scales).
    Returns (codes [G, T, D] u8, scales [G, T, D / block] float32).
    """
    x = bf16_bits_to_float(o_bits).astype(np.float32)
    T, H, Dh = x.shape
    cs = np.asarray(cos_sin_cache, dtype=np.float32)
    P, R = cs.shape
    assert R == rope_dim
    pos = np.asarray(positions, dtype=np.int64)
    ok = (pos >= 0) & (pos < P)
    pc = np.where(ok, pos, 0)
    rot = inv_rope_gptj_tail(x, cs[pc, : R // 2], cs[pc, R // 2:], R)
    hpg = H // n_groups
    D = hpg * Dh
    rows = rot.reshape(T, n_groups, D).transpose(1, 0, 2)  # [G, T, D]
    codes, scales = fp8_pow2_quant(rows.reshape(n_groups, T, D // block, block))
    codes = codes.reshape(n_groups, T, D)
    codes[:, ~ok] = 0
    scales[:, ~ok] = 0.0
    return codes, scales


# ---------------------------------------------------------------------------
# Cache write side: compressed KV rows and indexer keys into their paged caches
# ---------------------------------------------------------------------------


def compressed_position(positions, ratio: int) -> np.ndarray:
    """[ops] ``_fp8_ds_mla_cache_rows``: the RoPE position of a compressed row is its
    token position rounded down to a multiple of the compress ratio."""
    return (np.asarray(positions, dtype=np.int64) // ratio) * ratio


def encode_kv_nope(x: np.ndarray):
    """bf16-valued nope rows [n, Dn] -> (e4m3fn bytes [n, Dn], fp32 scales [n, Dn/64]).

    Per 64 elements ([ops] ``_fp8_ds_mla_cache_rows``: blocks of 64, amax clamped
    below at 1e-4), with the fp32 scale form of these caches: scale =
    float32(max(amax, 1e-4)) / 448 and code = e4m3(clamp(x / scale, +-448)), both
    divisions single float32 operations.
    """
    x = np.asarray(x, dtype=np.float32)
    n, dn = x.shape
    blocks = x.reshape(n, dn // 64, 64)
    amax = np.maximum(np.abs(blocks).max(axis=-1), np.float32(1.0e-4)).astype(np.float32)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    y = np.clip((blocks / scale[..., None]).astype(np.float32), -448.0, 448.0)
    return e4m3_encode(y.astype(np.float64)).reshape(n, dn), scale


def encode_kv_nope_ue8m0(x: np.ndarray):
    """bf16-valued nope rows [n, Dn] -> (e4m3fn bytes [n, Dn], scale bytes [n, 8]).

    [ops] ``_fp8_ds_mla_cache_rows`` (the pages' native record): per 64 values,
    exponent = ceil(log2(max(amax, 1e-4) / 448)), written exactly as the smallest
    integer e with 448 * 2^e >= max(amax, 1e-4); codes e4m3(clamp(x * 2^-e, +-448));
    scale byte = clamp(e + 127, 0, 255); the row's 8th scale byte is a zero pad.
    """
    x = np.asarray(x, dtype=np.float64)
    n, dn = x.shape
    blocks = x.reshape(n, dn // 64, 64)
    a = np.maximum(np.abs(blocks).max(axis=-1), float(np.float32(1.0e-4)))
    e = np.empty(a.shape, dtype=np.int64)
    for idx, v in np.ndenumerate(a):
        k = math.ceil(math.log2(v / 448.0))
        while 448.0 * 2.0 ** (k - 1) >= v:
            k -= 1
        while 448.0 * 2.0 ** k < v:
            k += 1
        e[idx] = k
    y = np.clip(blocks * np.ldexp(1.0, -e)[..., None], -448.0, 448.0)
    sb = np.zeros((n, 8), dtype=np.uint8)
    sb[:, : dn // 64] = np.clip(e + 127, 0, 255).astype(np.uint8)
    return e4m3_encode(y).reshape(n, dn), sb


def insert_kv_rows(kv_pages: dict, rows_bits, positions, cos_sin_cache, ratio: int, slots,
                   block_size: int, d_nope: int, d_rope: int, num_pages: int, page_bytes: int,
                   scale_format: str = "f32") -> dict:
    """Write compressed KV rows into the paged latent cache; returns the updated pages.

    [ops] ``_write_fp8_ds_mla_cache_rows_capturable`` / ``_fp8_ds_mla_cache_rows``:
    the rope tail is rotated (GPT-J) at the compressed position and stored bf16;
    the nope part is stored FP8 with one scale per 64 (``encode_kv_nope``); row
    ``o`` of page ``g`` holds its values at ``g*stride + o*(Dn + 2*Dr)`` and its
    scales at ``g*stride + B*(Dn + 2*Dr) + o*scale_bytes``.  In the native "ue8m0"
    form the nope part takes ``encode_kv_nope_ue8m0``.  A slot that is negative or
    whose page is past the pool is skipped.  Pages not yet in ``kv_pages`` start as
    zero bytes.
    """
    x = bf16_bits_to_float(rows_bits).astype(np.float32)
    cs = np.asarray(cos_sin_cache, dtype=np.float32)
    cp = compressed_position(positions, ratio)
    out = {k: v.copy() for k, v in kv_pages.items()}
    row_b = d_nope + 2 * d_rope
    sbytes = kv_scale_bytes(d_nope, scale_format)
    for i, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0 or s // block_size >= num_pages or not (0 <= cp[i] < cs.shape[0]):
            continue
        roped = rope_gptj_tail(x[i], cs[cp[i], : d_rope // 2], cs[cp[i], d_rope // 2:], d_rope)
        if scale_format == "f32":
            codes, scale = encode_kv_nope(x[i: i + 1, :d_nope])
            scale_row = scale[0].astype(np.float32).view(np.uint8)
        else:
            codes, sb8 = encode_kv_nope_ue8m0(x[i: i + 1, :d_nope])
            scale_row = sb8[0]
        g, o = int(s) // block_size, int(s) % block_size
        page = out.setdefault(g, np.zeros(page_bytes, dtype=np.uint8))
        page[o * row_b: o * row_b + d_nope] = codes[0]
        page[o * row_b + d_nope: (o + 1) * row_b] = float32_to_bf16_bits(roped[d_nope:]).view(np.uint8)
        sb = block_size * row_b + o * sbytes
        page[sb: sb + sbytes] = scale_row
    return out


def insert_index_keys(idx_pages: dict, keys_bits, positions, cos_sin_cache, ratio: int, slots,
                      block_size: int, dim: int, num_pages: int, page_bytes: int) -> dict:
    """Write compressed indexer keys into the paged MXFP4 cache; returns the updated pages.

    [ops] compressor path (``_apply_gptj_rope_tail_rows`` at the compressed
    position, then ``_deepseek_v4_hadamard_rotate``, then the quantizer) and
    ``write_deepseek_v4_indexer_mxfp4_cache`` (page = ``[B x dim/2 values]`` then
    ``[B x dim/32 e8m0]``).  The key takes the same RoPE -> bf16 -> rotation ->
    MXFP4 steps as the query in ``prepare_indexer_q_mxfp4``.  A slot that is
    negative or whose page is past the pool is skipped.
    """
    cs = np.asarray(cos_sin_cache, dtype=np.float32)
    R = cs.shape[1]
    cp = compressed_position(positions, ratio)
    out = {k: v.copy() for k, v in idx_pages.items()}
    vb, sb = dim // 2, dim // 32
    x = bf16_bits_to_float(keys_bits).astype(np.float32)
    for i, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0 or s // block_size >= num_pages or not (0 <= cp[i] < cs.shape[0]):
            continue
        roped = rope_gptj_tail(x[i], cs[cp[i], : R // 2], cs[cp[i], R // 2:], R)
        rotated = hadamard_rotate(float32_to_bf16_bits(roped))
        vals, exps = mxfp4_encode(bf16_bits_to_float(rotated)[None, :])
        g, o = int(s) // block_size, int(s) % block_size
        page = out.setdefault(g, np.zeros(page_bytes, dtype=np.uint8))
        page[o * vb: (o + 1) * vb] = vals[0]
        page[block_size * vb + o * sb: block_size * vb + (o + 1) * sb] = exps[0]
    return out


# ---------------------------------------------------------------------------
# Whole step
# ---------------------------------------------------------------------------


def step(view, cfg, padded_topk, kv_num_pages, idx_num_pages, softmax_scale, tokens=None, attn_sink=None,
         swa_num_pages=None):
    """Indexer -> top-k -> index build -> attention for one layer.

    ``view`` holds numpy inputs (see the workload host view); ``cfg`` gives
    the shape parameters.  The window rows are read from ``view.swa_pages`` with
    ``cfg.swa_block_size`` rows per page when the view has a window cache of its own
    (``swa_num_pages`` pages), else from the compressed rows' pages.  Returns a dict of
    every intermediate.
    """
    swa_pages = getattr(view, "swa_pages", None) or view.kv_pages
    swa_block = getattr(cfg, "swa_block_size", cfg.block)
    swa_num_pages = kv_num_pages if swa_num_pages is None else swa_num_pages
    T = len(view.token_to_req)
    all_tokens = list(range(T)) if tokens is None else list(tokens)
    if cfg.topk > 0:
        tk = np.full((T, cfg.topk), -1, np.int32)
        sel = indexer_topk(view.query_start_loc, view.seq_lens, view.token_to_req,
                           view.idx_q_values, view.idx_q_scales, view.idx_weights,
                           view.idx_pages, view.idx_bt, cfg.idx_block, cfg.idx_dim, idx_num_pages,
                           cfg.ratio, cfg.topk, tokens=all_tokens)
        tk[all_tokens] = sel
    else:
        tk = None
    si, lens = build_sparse_indices(
        view.query_start_loc, view.seq_lens, view.token_to_req, view.replay_start,
        view.swa_bt, swa_block, swa_num_pages, view.comp_bt, cfg.block, kv_num_pages,
        tk, cfg.topk, cfg.window, cfg.ratio, padded_topk)
    o, lse = sparse_mla_decode(view.q, swa_pages, view.kv_pages, si, lens, cfg.window,
                               swa_block, cfg.block, cfg.d_nope, cfg.d_rope, softmax_scale,
                               attn_sink=attn_sink, tokens=all_tokens,
                               scale_format=getattr(cfg, "kv_format", "f32"))
    return {"topk": tk, "sparse_indices": si, "lens": lens, "out": o, "lse": lse, "tokens": all_tokens}
