"""sparse_mla_decode_noalloc (no workspace: the split partials use the library's static
per-GPU scratch) against sparse_mla_decode, through the C ABI, on two calls in a row, the
second with a smaller input.

The first input splits each token's columns so that sparse_mla_decode's partials (16
splits, ~37.8 MB) exceed the 32 MiB scratch: the entry point then uses fewer splits,
which changes only the fp32 summation order.  Bar between the two outputs: max(5e-3, one
bf16 ulp of the larger value); lse within 1e-3."""

import numpy as np
import pytest
import torch

import sparse_attention_decode_build_amd as sad
from sparse_attention_decode_build_amd import workloads as WL

from gpu_helpers import ATOL_LSE, ATOL_OUT, bf16_to_f64, gpu_build, kv_caches, log

pytestmark = pytest.mark.gpu

# dense compressed path (ratio 128, every compressed row attended): 8 requests with 16384
# compressed rows each, then 4 requests with 2048
BIG = WL.with_overrides(WL.CONFIGS["dense_1m"], name="dense_2m_x8", groups=((8, 1, 1 << 21, 0),),
                        kv_pool_pages=0)
SMALL = WL.with_overrides(WL.CONFIGS["dense_1m"], name="dense_256k_x4", seed=7, groups=((4, 1, 1 << 18, 0),),
                          kv_pool_pages=0)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sad.load()
    yield
    torch.cuda.synchronize()


def _ulp(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def _compare(cfg):
    log(f"[case] no-alloc vs workspace entry point: {cfg.name}")
    wl = WL.make_workload(cfg, "cuda")
    c = wl.cfg
    T = wl.num_tokens
    si, lens = gpu_build(wl, None)
    swa, comp = kv_caches(wl)
    q = wl.layers[0].q
    width = c.window + wl.padded_topk
    need = sad.sparse_mla_decode_workspace_size(T, c.heads, width, c.dqk)
    lse_a = torch.empty((T, c.heads), dtype=torch.float32, device="cuda")
    lse_b = torch.full((T, c.heads), float("nan"), dtype=torch.float32, device="cuda")
    out_a = sad.sparse_mla_decode(q, swa, comp, si, lens, c.window, wl.padded_topk, wl.softmax_scale, lse=lse_a)
    out_b = torch.full_like(out_a, float("nan"))
    sad.sparse_mla_decode_noalloc(q, swa, comp, si, lens, c.window, wl.padded_topk, wl.softmax_scale, out=out_b,
                                  lse=lse_b)
    torch.cuda.synchronize()
    a, b = bf16_to_f64(out_a), bf16_to_f64(out_b)
    assert np.all(np.isfinite(b)), "every output written"
    err = np.abs(a - b)
    bar = np.maximum(ATOL_OUT, _ulp(np.maximum(np.abs(a), np.abs(b))))
    log(f"[report] {cfg.name}: T={T}, workspace entry point needs {need} bytes; max |diff| {err.max():.3e}, "
        f"{int((err > 0).sum())} of {err.size} elements differ")
    assert np.all(err <= bar)
    la, lb = lse_a.cpu().numpy(), lse_b.cpu().numpy()
    assert np.max(np.abs(la - lb)) <= ATOL_LSE
    del wl
    torch.cuda.empty_cache()
    return need


def test_noalloc_matches_the_workspace_entry_point_twice():
    need_big = _compare(BIG)
    assert need_big > 32 << 20, "the first input must exceed the scratch (the split cap engages)"
    need_small = _compare(SMALL)
    assert 0 < need_small < need_big, "the second input is smaller and still split"
