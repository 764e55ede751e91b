"""libsad.so loads, exports every function include/sad.h declares, and rejects bad
arguments on the host (no kernel launch, so these run without a GPU)."""

import ctypes
import os
import re
import subprocess

import pytest

from sparse_attention_decode_build_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from sparse_attention_decode_build_amd.build import build

        build()
    return L.load()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "sad.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert {"build_sparse_indices", "indexer_score_topk", "gather_dequant_kv", "sparse_mla_decode"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


FAKE = 4096  # a non-NULL, 16-byte aligned pointer value that is never dereferenced on the host


def _batch(T, R=1):
    return L.SadBatch(FAKE, FAKE, FAKE, R, T)


def _kv(d_nope=512, d_rope=64, block=64, stride=None, pages=10):
    stride = stride if stride is not None else block * (d_nope + 2 * d_rope + 4 * (d_nope // 64))
    return L.SadKvCache(FAKE, stride, pages, block, d_nope, d_rope)


def _call_build(lib, batch, padded=64, topk=16, window=32, stride=16, ratio=4):
    return lib.build_sparse_indices(
        ctypes.byref(batch) if batch is not None else None, None, FAKE, 4, 4, 16, 100, FAKE, 4, 4, 16,
        100, FAKE, stride, topk, window, ratio, padded, FAKE, FAKE, None)


def test_build_sparse_indices_errors(lib):
    assert _call_build(lib, None) == L.SAD_EINVAL
    assert "batch" in L.last_error()
    assert _call_build(lib, _batch(0)) == L.SAD_OK  # empty batch: no launch
    assert L.last_error() == ""
    assert _call_build(lib, _batch(3), padded=60) == L.SAD_EINVAL  # not a multiple of 64
    assert _call_build(lib, _batch(3), topk=128, padded=64) == L.SAD_EINVAL  # topk > padded
    assert _call_build(lib, _batch(3), stride=8) == L.SAD_EINVAL  # topk_stride < topk
    assert _call_build(lib, _batch(3), ratio=0) == L.SAD_EINVAL
    assert _call_build(lib, _batch(-1)) == L.SAD_EINVAL


def _call_indexer(lib, T=2, dim=128, heads=64, block=64, cols=4, topk=16, ws_bytes=1 << 30, ratio=4):
    keys = L.SadMxfp4Cache(FAKE, block * (dim // 2 + dim // 32), 10, block, dim)
    b = _batch(T)
    return lib.indexer_score_topk(ctypes.byref(b), FAKE, FAKE, FAKE, heads, ctypes.byref(keys), FAKE,
                                  cols, cols, ratio, topk, FAKE, None, 0, FAKE, ws_bytes, None)


def test_indexer_errors(lib):
    assert _call_indexer(lib, T=0) == L.SAD_OK
    assert _call_indexer(lib, dim=96) == L.SAD_EUNSUPPORTED
    assert _call_indexer(lib, heads=65) == L.SAD_EUNSUPPORTED
    assert _call_indexer(lib, block=32) == L.SAD_EUNSUPPORTED
    # 1M rows: 32 chunks of 32768 rows x topk 2048 candidates > 32768
    assert _call_indexer(lib, cols=16384, topk=2048) == L.SAD_EUNSUPPORTED
    assert "chunks" in L.last_error()
    assert _call_indexer(lib, topk=0) == L.SAD_EINVAL
    assert _call_indexer(lib, ws_bytes=16) == L.SAD_EWORKSPACE
    assert "workspace" in L.last_error()
    need = lib.indexer_score_topk_workspace_size(128, 16384, 2048)
    assert need == 128 * 16384 * 4
    # past 32768 rows: the logits plus the chunks' candidates (value and row id)
    assert lib.indexer_score_topk_workspace_size(128, 262144, 2048) == 128 * 262144 * 4 + 2 * 128 * 8 * 2048 * 4
    assert lib.indexer_score_topk_workspace_size(0, 16384, 2048) == 0


def test_gather_errors(lib):
    s, c = _kv(), _kv()
    assert lib.gather_dequant_kv(ctypes.byref(s), ctypes.byref(c), FAKE, FAKE, 0, 128, 2048, FAKE, None) == L.SAD_OK
    bad = _kv(d_nope=256)
    assert lib.gather_dequant_kv(ctypes.byref(bad), ctypes.byref(c), FAKE, FAKE, 4, 128, 2048, FAKE, None) == L.SAD_EUNSUPPORTED
    small = _kv(stride=1024)
    assert lib.gather_dequant_kv(ctypes.byref(small), ctypes.byref(c), FAKE, FAKE, 4, 128, 2048, FAKE, None) == L.SAD_EINVAL
    tiny = _kv(d_nope=128, d_rope=32, block=16)
    assert lib.gather_dequant_kv(ctypes.byref(tiny), ctypes.byref(c), FAKE, FAKE, 4, 128, 2048, FAKE, None) == L.SAD_EINVAL
    huge = _kv(pages=1 << 30)
    assert lib.gather_dequant_kv(ctypes.byref(huge), ctypes.byref(c), FAKE, FAKE, 4, 128, 2048, FAKE, None) == L.SAD_EINVAL


def _call_attn(lib, T=128, H=128, ws=None, ws_bytes=0, W=128, P=2048):
    s, c = _kv(), _kv()
    return lib.sparse_mla_decode(FAKE, T, H, ctypes.byref(s), ctypes.byref(c), FAKE, FAKE, W, P, 0.04, None,
                                 FAKE, None, ws, ws_bytes, None)


def test_attention_errors(lib):
    assert _call_attn(lib, T=0) == L.SAD_OK
    assert _call_attn(lib, H=7) == L.SAD_EUNSUPPORTED
    assert _call_attn(lib, H=256) == L.SAD_EUNSUPPORTED
    # few tokens -> split columns -> partials need a workspace
    need = lib.sparse_mla_decode_workspace_size(8, 128, 128 + 8192, 576)
    assert need > 0
    assert _call_attn(lib, T=8, P=8192) == L.SAD_EWORKSPACE
    assert "workspace" in L.last_error()
    assert lib.sparse_mla_decode_workspace_size(16448, 128, 2176, 576) == 0


def _call_attn_noalloc(lib, T=128, H=128, W=128, P=2048, d_nope=512):
    s, c = _kv(d_nope=d_nope), _kv(d_nope=d_nope)
    return lib.sparse_mla_decode_noalloc(FAKE, T, H, ctypes.byref(s), ctypes.byref(c), FAKE, FAKE, W, P, 0.04,
                                         None, FAKE, None, None)


def test_attention_noalloc_errors(lib):
    """The entry point for callers that cannot allocate checks its arguments as
    sparse_mla_decode does; it never asks for a workspace."""
    assert _call_attn_noalloc(lib, T=0) == L.SAD_OK
    assert L.last_error() == ""
    assert _call_attn_noalloc(lib, H=7) == L.SAD_EUNSUPPORTED
    assert "sparse_mla_decode_noalloc" in L.last_error()
    assert _call_attn_noalloc(lib, T=-1) == L.SAD_EINVAL
    assert _call_attn_noalloc(lib, T=70000) == L.SAD_EINVAL
    assert _call_attn_noalloc(lib, d_nope=256) == L.SAD_EUNSUPPORTED


def _call_qprep(lib, T=4, H=64, D=128, R=64, P=100, align=FAKE):
    return lib.prepare_indexer_q_mxfp4(align, FAKE, FAKE, P, R, FAKE, 0.088, 0.125, T, H, D,
                                       FAKE, FAKE, FAKE, None)


def test_prepare_indexer_q_errors(lib):
    assert _call_qprep(lib, T=0) == L.SAD_OK
    assert _call_qprep(lib, D=96) == L.SAD_EUNSUPPORTED
    assert _call_qprep(lib, R=0) == L.SAD_EINVAL
    assert _call_qprep(lib, R=128) == L.SAD_EINVAL  # not below idx_dim
    assert _call_qprep(lib, R=36) == L.SAD_EINVAL  # not a multiple of 8
    assert _call_qprep(lib, P=0) == L.SAD_EINVAL
    assert _call_qprep(lib, T=-1) == L.SAD_EINVAL
    assert _call_qprep(lib, align=FAKE + 4) == L.SAD_EINVAL
    assert "aligned" in L.last_error()


def _call_outq(lib, T=4, H=128, Dh=576, R=64, G=16, P=100, align=FAKE):
    return lib.inv_rope_fp8_quant(align, FAKE, FAKE, P, R, T, H, Dh, G, FAKE, FAKE, None)


def test_inv_rope_fp8_quant_errors(lib):
    assert _call_outq(lib, T=0) == L.SAD_OK
    assert _call_outq(lib, G=3) == L.SAD_EINVAL  # 128 heads not a multiple of 3
    assert _call_outq(lib, R=0) == L.SAD_EINVAL
    assert _call_outq(lib, R=36) == L.SAD_EINVAL
    assert _call_outq(lib, R=640) == L.SAD_EINVAL  # rope longer than the head
    assert _call_outq(lib, H=2, G=2, Dh=72, R=8) == L.SAD_EINVAL  # D = 72 not a multiple of 128
    assert _call_outq(lib, H=16, G=1, Dh=24, R=8) == L.SAD_EINVAL  # head_dim below 32
    assert _call_outq(lib, P=0) == L.SAD_EINVAL
    assert _call_outq(lib, align=FAKE + 8) == L.SAD_EINVAL
    assert "aligned" in L.last_error()


def test_insert_kv_rows_errors(lib):
    c = _kv()
    ok = lambda **k: lib.insert_kv_rows(k.get("rows", FAKE), FAKE, FAKE, k.get("P", 100), k.get("ratio", 4), FAKE,
                                        k.get("N", 3), ctypes.byref(k.get("cache", c)), None)
    assert ok(N=0) == L.SAD_OK
    assert ok(ratio=0) == L.SAD_EINVAL
    assert ok(P=0) == L.SAD_EINVAL
    assert ok(rows=FAKE + 2) == L.SAD_EINVAL
    assert ok(cache=_kv(d_nope=256)) == L.SAD_EUNSUPPORTED
    assert ok(cache=_kv(stride=1024)) == L.SAD_EINVAL
    assert lib.insert_kv_rows(FAKE, FAKE, FAKE, 100, 4, FAKE, 3, None, None) == L.SAD_EINVAL


def test_insert_index_keys_errors(lib):
    def call(dim=128, block=64, R=64, N=3, P=100, ratio=4, stride=None):
        stride = stride if stride is not None else block * (dim // 2 + dim // 32)
        keys = L.SadMxfp4Cache(FAKE, stride, 10, block, dim)
        return lib.insert_index_keys(FAKE, FAKE, FAKE, P, R, ratio, FAKE, N, ctypes.byref(keys), None)
    assert call(N=0) == L.SAD_OK
    assert call(dim=96) == L.SAD_EUNSUPPORTED
    assert call(block=32) == L.SAD_EUNSUPPORTED
    assert call(R=128) == L.SAD_EINVAL
    assert call(ratio=0) == L.SAD_EINVAL
    assert call(stride=64) == L.SAD_EINVAL
    assert call(P=0) == L.SAD_EINVAL


def test_indexer_topk_sparse_indices_errors(lib):
    keys = L.SadMxfp4Cache(FAKE, 64 * 68, 10, 64, 128)

    def call(T=2, padded=2048, topk=2048, dim=128, window=128, ratio=4):
        k = keys if dim == 128 else L.SadMxfp4Cache(FAKE, 64 * 68, 10, 64, dim)
        b = _batch(T)
        return lib.indexer_topk_sparse_indices(ctypes.byref(b), FAKE, FAKE, FAKE, 64, ctypes.byref(k), FAKE, 4, 4,
                                               ratio, topk, FAKE, None, FAKE, 4, 4, 64, 100, FAKE, 4, 4, 64, 100,
                                               window, padded, FAKE, FAKE, FAKE, 1 << 30, None)
    assert call(T=0) == L.SAD_OK
    assert call(padded=2000) == L.SAD_EINVAL  # not a multiple of 64
    assert call(topk=4096) == L.SAD_EINVAL  # topk > padded
    assert "indexer_topk_sparse_indices" in L.last_error()
    assert call(dim=96) == L.SAD_EUNSUPPORTED
    assert call(ratio=0) == L.SAD_EINVAL
