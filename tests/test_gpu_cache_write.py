"""GPU parity of the cache write side (insert_kv_rows, insert_index_keys) against the CPU
oracle: the same seeded rows are written into pools of random bytes, and every page of
the pool is compared byte for byte (written rows, their scales, and untouched bytes).

Bar: bit-exact.  The codes and scales are integers and floats decided by floating point;
both sides take every decision with the same correctly rounded fp32 operations.
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


def _slots(n, pages, block, seed):
    g = np.random.default_rng(seed)
    s = g.choice(pages * block, size=n, replace=False).astype(np.int64)
    s[::7] = -1                       # skipped
    if n > 3:
        s[3] = pages * block + 5      # page past the pool: skipped
    return s


@pytest.mark.parametrize("Dn,Dr,B,N,ratio,fmt", [(512, 64, 64, 37, 4, "f32"), (128, 32, 16, 20, 4, "f32"),
                                                (512, 64, 64, 2048, 128, "f32"), (448, 64, 64, 45, 4, "ue8m0"),
                                                (448, 64, 16, 900, 128, "ue8m0")])
def test_insert_kv_rows_pages_bit_exact(Dn, Dr, B, N, ratio, fmt):
    log(f"[kvw] Dn={Dn} Dr={Dr} B={B} N={N} ratio={ratio} {fmt}")
    pages, P = 64, 3000
    row_b = Dn + 2 * Dr
    page_bytes = B * (row_b + O.kv_scale_bytes(Dn, fmt))
    g = torch.Generator().manual_seed(N)
    pool = torch.randint(0, 256, (pages, page_bytes), dtype=torch.uint8, generator=g)
    rows = (torch.randn(N, Dn + Dr, generator=g) * torch.exp2(torch.randint(-6, 6, (N, 1), generator=g).float())).bfloat16()
    rows[1] = 0
    pos = torch.randint(0, P + 40, (N,), generator=g, dtype=torch.int32)  # some outside the table
    slots = _slots(N, pages, B, N)
    cs = WL.rope_table(P, Dr)
    before = {p: pool[p].numpy().copy() for p in range(pages)}
    dev_pool = pool.cuda()
    kv = sad.KvCache(dev_pool, B, Dn, Dr, sad.KV_SCALE_UE8M0 if fmt == "ue8m0" else sad.KV_SCALE_F32)
    sad.insert_kv_rows(rows.cuda(), pos.cuda(), cs.cuda(), ratio, torch.from_numpy(slots.astype(np.int32)).cuda(), kv)
    torch.cuda.synchronize()
    want = O.insert_kv_rows(before, _bits(rows), pos.numpy(), cs.numpy(), ratio, slots, B, Dn, Dr, pages,
                            page_bytes, fmt)
    got = dev_pool.cpu().numpy()
    for p in range(pages):
        bad = np.flatnonzero(got[p] != want[p])
        assert bad.size == 0, f"page {p}: {bad.size} bytes differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("D,R,B,N,ratio", [(128, 64, 64, 41, 4), (64, 32, 16, 9, 4), (128, 64, 64, 2048, 4)])
def test_insert_index_keys_pages_bit_exact(D, R, B, N, ratio):
    log(f"[idxw] D={D} R={R} B={B} N={N} ratio={ratio}")
    pages, P = 48, 5000
    page_bytes = B * (D // 2 + D // 32)
    g = torch.Generator().manual_seed(N + 1)
    pool = torch.randint(0, 256, (pages, page_bytes), dtype=torch.uint8, generator=g)
    keys = torch.randn(N, D, generator=g).bfloat16()
    keys[2] = 0
    pos = torch.randint(0, P + 60, (N,), generator=g, dtype=torch.int32)
    slots = _slots(N, pages, B, N + 1)
    cs = WL.rope_table(P, R)
    before = {p: pool[p].numpy().copy() for p in range(pages)}
    dev_pool = pool.cuda()
    idx = sad.IndexerCache(dev_pool, B, D)
    sad.insert_index_keys(keys.cuda(), pos.cuda(), cs.cuda(), ratio, torch.from_numpy(slots.astype(np.int32)).cuda(), idx)
    torch.cuda.synchronize()
    want = O.insert_index_keys(before, _bits(keys), pos.numpy(), cs.numpy(), ratio, slots, B, D, pages, page_bytes)
    got = dev_pool.cpu().numpy()
    for p in range(pages):
        bad = np.flatnonzero(got[p] != want[p])
        assert bad.size == 0, f"page {p}: {bad.size} bytes differ, first at {bad[:4].tolist()}"


def test_written_keys_score_like_prepared_queries():
    # A key written by insert_index_keys and the same vector prepared as a query at
    # the same (compressed) position carry identical codes: both take the same steps.
    D, R, B, P = 128, 64, 64, 256
    g = torch.Generator().manual_seed(77)
    v = torch.randn(4, D, generator=g).bfloat16().cuda()
    pos = torch.tensor([8, 9, 64, 200], dtype=torch.int32).cuda()
    cs = WL.rope_table(P, R).cuda()
    pool = torch.zeros((1, B * (D // 2 + D // 32)), dtype=torch.uint8).cuda()
    sad.insert_index_keys(v, pos, cs, 4, torch.arange(4, dtype=torch.int32).cuda(), sad.IndexerCache(pool, B, D))
    cp = (pos // 4) * 4
    qv, qs, _ = sad.prepare_indexer_q_mxfp4(v[:, None, :].contiguous(), cp, cs,
                                            torch.ones(4, 1).cuda(), 1.0, 1.0)
    torch.cuda.synchronize()
    page = pool[0].cpu()
    assert torch.equal(page[: 4 * D // 2].view(4, D // 2), qv[:, 0].cpu())
    assert torch.equal(page[B * D // 2: B * D // 2 + 4 * D // 32].view(4, D // 32), qs[:, 0].cpu())
