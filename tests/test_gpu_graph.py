"""The fused step (indexer_topk_sparse_indices, then sparse_mla_decode) captured into a HIP
graph: no entry point allocates, syncs or clears memory with a memset, so the step can be
captured.  The graph is replayed several times with other eager work and synchronizations
between the replays, and every replay's outputs must equal the eager step's bit for bit."""

import pytest
import torch

import sparse_attention_decode_build_amd as sad
from sparse_attention_decode_build_amd import workloads as WL

from gpu_helpers import free, idx_cache, kv_caches, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sad.load()
    yield


def _step(wl, layer, outs, stream):
    c = wl.cfg
    L = wl.layers[layer]
    swa, comp = kv_caches(wl)
    topk, si, lens, out, ws_i, ws_a = outs
    sad.indexer_topk_sparse_indices(
        wl.query_start_loc, wl.seq_lens, wl.token_to_req, L.idx_q_values, L.idx_q_scales, L.idx_weights,
        idx_cache(wl), L.idx_bt, c.ratio, c.topk, wl.replay_start, L.swa_bt, c.swa_block_size,
        wl.swa_pool.shape[0], L.comp_bt, c.block, wl.kv_pool.shape[0], c.window, wl.padded_topk,
        topk_local=topk, out=si, lens=lens, workspace=ws_i, stream=stream)
    sad.sparse_mla_decode(L.q, swa, comp, si, lens, c.window, wl.padded_topk, wl.softmax_scale, out=out,
                          workspace=ws_a, stream=stream)


def _outs(wl):
    c, T, dev = wl.cfg, wl.num_tokens, wl.device
    max_rows = wl.layers[0].idx_bt.shape[1] * c.idx_block
    ws_i = torch.empty((max(sad.indexer_score_topk_workspace_size(T, max_rows, c.topk), 16),),
                       dtype=torch.uint8, device=dev)
    ws_a = torch.empty((max(sad.sparse_mla_decode_workspace_size(T, c.heads, c.window + wl.padded_topk, c.dqk),
                            16),), dtype=torch.uint8, device=dev)
    return (torch.empty((T, c.topk), dtype=torch.int32, device=dev),
            torch.empty((T, c.window + wl.padded_topk), dtype=torch.int32, device=dev),
            torch.empty((T,), dtype=torch.int32, device=dev),
            torch.empty((T, c.heads, c.dqk), dtype=torch.bfloat16, device=dev), ws_i, ws_a)


@pytest.mark.parametrize("name", ["tiny", "b32_8k", "two_cache_b8_8k"])
def test_graph_replays_equal_the_eager_step(name):
    log(f"[graph] {name}")
    wl = WL.make_workload(name, "cuda", num_layers=2)
    s = torch.cuda.Stream()
    outs = _outs(wl)
    other = _outs(wl)
    with torch.cuda.stream(s):
        _step(wl, 0, outs, s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs[:4]]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _step(wl, 0, outs, s)
    for rep in range(3):
        for t in outs[:4]:
            t.zero_()
        with torch.cuda.stream(s):
            _step(wl, 1, other, s)  # eager work of another layer between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs[:4], ref):
            assert torch.equal(a, b), f"replay {rep} differs"
    del g
    free(wl)
