"""Benchmark of the sparse-attention decode step on one MI355X.

A step is one pass of the whole hot path over one batch: indexer_score_topk (MXFP4
scoring + top-k) -> build_sparse_indices -> sparse_mla_decode (fused gather + FP8
dequant + MLA attention), all through the C ABI of libsad.so on one HIP stream.

Workload: 128 requests x 1 decode token at 64K context (window 128, compress ratio 4
-> 16384 compressed rows, top-2048, 128 heads, latent 512 FP8 + 64 bf16, indexer 64
heads x 128 MXFP4, page size 64), pages shuffled over a ~196 GB KV pool and a ~3.9 GB
indexer pool.  Several independent layers (own pages, queries and tables) are
rotated step by step so the 256 MB MALL cannot serve a step from the previous one.
Inputs are resident in HBM before timing starts.

Prints one JSON line (rank 0) with tokens/s, per-kernel times, roofline objects for
the attention kernel (HBM and MFMA views) and the CPU oracle's throughput on a
bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_attention_decode_build_amd as sad  # noqa: E402
from sparse_attention_decode_build_amd import _lib as L  # noqa: E402
from sparse_attention_decode_build_amd import workloads as WL  # noqa: E402

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
WORKLOAD = WL.HEADLINE
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "counters_b128_64k.md")
# the headline attention kernel (512 fp8 + 64 bf16 latent rows) and its source file
ATTN_KERNEL = "mla_dsplit_kernel"
ATTN_SRC = "attention_dsplit.hip"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Step:
    """Pre-marshalled C-ABI calls for one layer (no Python work in the timed loop)."""

    def __init__(self, wl: WL.Workload, layer: int, stream=None):
        cfg = wl.cfg
        lay = wl.layers[layer]
        self.lib = L.load()
        T, dev = wl.num_tokens, wl.device
        self.batch = L.SadBatch(wl.query_start_loc.data_ptr(), wl.seq_lens.data_ptr(),
                                wl.token_to_req.data_ptr(), wl.num_reqs, T)
        self.kv = L.SadKvCache(wl.kv_pool.data_ptr(), wl.kv_pool.stride(0), wl.kv_pool.shape[0],
                               cfg.block, cfg.d_nope, cfg.d_rope, WL.kv_scale_format(cfg))
        self.idx = L.SadMxfp4Cache(wl.idx_pool.data_ptr(), wl.idx_pool.stride(0), wl.idx_pool.shape[0],
                                   cfg.idx_block, cfg.idx_dim)
        self.dense = cfg.dense
        self.topk = torch.empty((T, max(cfg.topk, 1)), dtype=torch.int32, device=dev)
        self.si = torch.empty((T, cfg.window + wl.padded_topk), dtype=torch.int32, device=dev)
        self.lens = torch.empty((T,), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, cfg.heads, cfg.dqk), dtype=torch.bfloat16, device=dev)
        max_rows = lay.idx_bt.shape[1] * cfg.idx_block
        ws_i = self.lib.indexer_score_topk_workspace_size(T, max_rows, cfg.topk)
        self.ws_i = torch.empty((max(ws_i, 16),), dtype=torch.uint8, device=dev)
        ws_a = self.lib.sparse_mla_decode_workspace_size(T, cfg.heads, cfg.window + wl.padded_topk, cfg.dqk)
        self.ws_a = torch.empty((max(ws_a, 16),), dtype=torch.uint8, device=dev)
        stream = ctypes.c_void_p((stream if stream is not None else torch.cuda.current_stream()).cuda_stream)
        p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        n_pages = wl.kv_pool.shape[0]
        self.args_idx = (ctypes.byref(self.batch), p(lay.idx_q_values), p(lay.idx_q_scales),
                         p(lay.idx_weights), cfg.idx_heads, ctypes.byref(self.idx), p(lay.idx_bt),
                         lay.idx_bt.stride(0), lay.idx_bt.shape[1], cfg.ratio, cfg.topk, p(self.topk),
                         None, 0, p(self.ws_i), self.ws_i.numel(), stream)
        self.args_build = (ctypes.byref(self.batch), p(wl.replay_start), p(lay.swa_bt), lay.swa_bt.stride(0),
                           lay.swa_bt.shape[1], cfg.block, n_pages, p(lay.comp_bt), lay.comp_bt.stride(0),
                           lay.comp_bt.shape[1], cfg.block, n_pages, None if self.dense else p(self.topk),
                           self.topk.stride(0), cfg.topk, cfg.window, cfg.ratio, wl.padded_topk, p(self.si),
                           p(self.lens), stream)
        self.args_fused = (ctypes.byref(self.batch), p(lay.idx_q_values), p(lay.idx_q_scales),
                           p(lay.idx_weights), cfg.idx_heads, ctypes.byref(self.idx), p(lay.idx_bt),
                           lay.idx_bt.stride(0), lay.idx_bt.shape[1], cfg.ratio, cfg.topk, p(self.topk),
                           p(wl.replay_start), p(lay.swa_bt), lay.swa_bt.stride(0), lay.swa_bt.shape[1],
                           cfg.block, n_pages, p(lay.comp_bt), lay.comp_bt.stride(0), lay.comp_bt.shape[1],
                           cfg.block, n_pages, cfg.window, wl.padded_topk, p(self.si), p(self.lens),
                           p(self.ws_i), self.ws_i.numel(), stream)
        self.args_attn = (p(lay.q), T, cfg.heads, ctypes.byref(self.kv), ctypes.byref(self.kv), p(self.si),
                          p(self.lens), cfg.window, wl.padded_topk, ctypes.c_float(wl.softmax_scale), None,
                          p(self.out), None, p(self.ws_a), self.ws_a.numel(), stream)

    def run(self, ev=None, fused=True):
        """One step: the indexer, top-k and index build (one call, or two when not fused),
        then the attention.  ev (optional): [after the indexer call (two-call step only),
        just before the attention, just after it], each an event or None.  Each record
        costs the step a few microseconds, so no event precedes the indexer: its segment
        is taken from the previous step's last event."""
        lib = self.lib
        ev = ev if ev is not None else [None, None, None]
        if self.dense:  # every compressed row attended: no indexer
            rc = lib.build_sparse_indices(*self.args_build)
        elif fused:
            rc = lib.indexer_topk_sparse_indices(*self.args_fused)
        else:
            rc = lib.indexer_score_topk(*self.args_idx)
            if ev[0] is not None:
                ev[0].record()
            rc |= lib.build_sparse_indices(*self.args_build)
        if ev[1] is not None:
            ev[1].record()
        rc |= lib.sparse_mla_decode(*self.args_attn)
        if ev[2] is not None:
            ev[2].record()
        if rc:
            raise RuntimeError(f"step failed: {L.last_error()}")


def algorithmic_bytes(wl: WL.Workload) -> dict:
    """Bytes the method must move per step (each FP8/MXFP4 row once, q, out, indices)."""
    cfg = wl.cfg
    seq = wl.seq_lens.cpu().numpy().astype(np.int64)
    qsl = wl.query_start_loc.cpu().numpy().astype(np.int64)
    t2r = wl.token_to_req.cpu().numpy().astype(np.int64)
    pos = seq[t2r] - (qsl[t2r + 1] - qsl[t2r]) + (np.arange(len(t2r)) - qsl[t2r])
    nc = (pos + 1) // cfg.ratio
    # attended rows per token: the window, then the top-k (dense: every compressed row)
    rows = np.minimum(pos + 1, cfg.window) + (nc if cfg.dense else np.minimum(nc, cfg.topk))
    row_b = cfg.d_nope + 2 * cfg.d_rope + cfg.kv_scale_bytes
    idx_row = cfg.idx_dim // 2 + cfg.idx_dim // 32
    W, P, H, D = cfg.window, wl.padded_topk, cfg.heads, cfg.dqk
    attn = rows * row_b + (W + P) * 4 + 4 + 2 * H * D + 2 * H * D
    indexer = (nc * idx_row + (nc + cfg.idx_block - 1) // cfg.idx_block * 4
               + cfg.idx_heads * idx_row + 4 * cfg.idx_heads + 4 * cfg.topk) * (0 if cfg.dense else 1)
    build = 4 * cfg.topk + 4 * (W + P)
    flops = 2 * H * (D + D) * rows  # QK + PV
    return {"attention": int(attn.sum()), "indexer": int(indexer.sum()), "build": int(build * len(t2r)),
            "attention_flops": int(flops.sum()), "rows": int(rows.sum())}


def measured_traffic():
    """HBM bytes per attention launch from committed rocprofv3 PMC runs, or None when
    the kernel source changed since they were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    src = open(os.path.join(ROOT, "sparse_attention_decode_build_amd", "csrc", ATTN_SRC), "rb").read()
    sha = hashlib.sha256(src).hexdigest()
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get(f"{ATTN_SRC} sha256") != sha:
        return None
    try:
        return float(vals["attention bytes per launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl: WL.Workload, budget_s: float) -> dict:
    """The CPU oracle, as it stands, on the first tokens of layer 0 (whole step each)."""
    from threadpoolctl import threadpool_info

    from oracle import sad_oracle as O

    cfg = wl.cfg
    T = wl.num_tokens

    def run(layer, tokens):
        view = WL.host_view(wl, layer, reqs=wl.token_to_req[tokens].cpu().tolist())
        t0 = time.perf_counter()
        O.step(view, cfg, wl.padded_topk, wl.kv_pool.shape[0], wl.idx_pool.shape[0], wl.softmax_scale,
               tokens=tokens)
        return time.perf_counter() - t0

    t1 = run(0, [0])
    n = int(min(T, max(2, budget_s / max(t1, 1e-3))))
    tokens = list(range(n))
    # whole steps of the rotated layers in turn while the budget lasts (one at least)
    done, total = 0, 0.0
    while done < len(wl.layers):
        dt = run(done, tokens)
        done += 1
        total += dt
        if n < T or total + dt > budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": done * n / total, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"whole step (indexer, top-k, index build, attention) of tokens 0..{n - 1} "
                      f"of layers 0..{done - 1} of the same {WORKLOAD} workload, float64 numpy oracle, "
                      f"{total:.1f} s"}


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(directory: str, suffix: str) -> str:
    for root, _, files in os.walk(directory):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {directory}")


def summarize_stats(directory: str) -> int:
    """Markdown table of a rocprofv3 --kernel-trace --stats --output-format csv run."""
    rows = _read_csv(_find(directory, "kernel_stats.csv"))
    print("| kernel | calls | average (us) | min (us) | max (us) |")
    print("|---|---|---|---|---|")
    other_calls, other_ns = 0, 0.0
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "").replace("void ", "")
        if not name.startswith("sad::"):  # torch kernels of the workload generator
            other_calls += int(r["Calls"])
            other_ns += float(r["TotalDurationNs"])
            continue
        print(f"| `{name.split('(')[0]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    print(f"| other (workload generation, torch) | {other_calls} | total {other_ns / 1e3:.0f} us | | |")
    return 0


def summarize_trace(directory: str) -> int:
    """Per-layer step of a rocprofv3 --kernel-trace run: for each occurrence of the fused
    step's kernel sequence (scoring, fused top-k + build, attention), the medians of the
    three kernels' durations and of the gaps between the end of one kernel and the start
    of the next (the attention's to the next scoring)."""
    import statistics
    rows = sorted(_read_csv(_find(directory, "kernel_trace.csv")), key=lambda r: int(r["Start_Timestamp"]))
    seq = ("indexer_score_kernel", "topk_kernel<16, 1>", ATTN_KERNEL)
    dur = {k: [] for k in seq}
    gaps = {"scoring -> top-k": [], "top-k -> attention": [], "attention -> next scoring": []}
    for i in range(len(rows) - 2):
        a, b, c = rows[i], rows[i + 1], rows[i + 2]
        if not all(k in r["Kernel_Name"] for k, r in zip(seq, (a, b, c))):
            continue
        for k, r in zip(seq, (a, b, c)):
            dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        gaps["scoring -> top-k"].append((int(b["Start_Timestamp"]) - int(a["End_Timestamp"])) / 1e3)
        gaps["top-k -> attention"].append((int(c["Start_Timestamp"]) - int(b["End_Timestamp"])) / 1e3)
        if i + 3 < len(rows) and seq[0] in rows[i + 3]["Kernel_Name"]:
            gaps["attention -> next scoring"].append((int(rows[i + 3]["Start_Timestamp"]) -
                                                      int(c["End_Timestamp"])) / 1e3)
    n = len(dur[seq[0]])
    print(f"{n} occurrences of the fused step's kernel sequence\n")
    print("| kernel or gap | median (us) |")
    print("|---|---|")
    for k, v in list(dur.items()) + list(gaps.items()):
        if v:
            print(f"| {k} | {statistics.median(v):.2f} |")
    return 0


# kernels of the step whose counters are summarized, and how their names start
COUNTER_KERNELS = (("attention", ATTN_KERNEL), ("indexer scoring", "indexer_score_kernel"),
                   ("top-k", "topk_kernel"))


def summarize_counters(dirs) -> int:
    """Markdown summary of rocprofv3 --pmc runs (one counter set per directory): for each
    step kernel, the mean value per dispatch of every counter, then the derived figures
    (MFMA busy share, bf16 / fp4 MFMA FLOPs, LDS bank-conflict share, HBM bytes from the
    request counts by size)."""
    vals = {}
    for d in dirs:
        if not os.path.isdir(d):
            continue
        for r in _read_csv(_find(d, "counter_collection.csv")):
            name = r["Kernel_Name"]
            for key, pat in COUNTER_KERNELS:
                if pat in name:
                    vals.setdefault(key, {}).setdefault(r["Counter_Name"], {}).setdefault(
                        r.get("Dispatch_Id", ""), 0.0)
                    vals[key][r["Counter_Name"]][r.get("Dispatch_Id", "")] += float(r["Counter_Value"])
    src = open(os.path.join(ROOT, "sparse_attention_decode_build_amd", "csrc", ATTN_SRC), "rb").read()
    print(f"- {ATTN_SRC} sha256: `{hashlib.sha256(src).hexdigest()}`\n")
    for key, _ in COUNTER_KERNELS:
        if key not in vals:
            continue
        m = {c: sum(v.values()) / len(v) for c, v in vals[key].items()}
        n = {c: len(v) for c, v in vals[key].items()}
        print(f"### {key}\n")
        print("| counter | mean per dispatch | dispatches |")
        print("|---|---|---|")
        for c in sorted(m):
            print(f"| `{c}` | {m[c]:.6g} | {n[c]} |")
        print()
        g = m.get
        if g("SQ_BUSY_CU_CYCLES") and g("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
            print(f"- MFMA busy: {100 * g('SQ_VALU_MFMA_BUSY_CYCLES') / (4 * g('SQ_BUSY_CU_CYCLES')):.1f}% of the "
                  "SIMD cycles of busy CUs (SQ_VALU_MFMA_BUSY_CYCLES / (4 x SQ_BUSY_CU_CYCLES))")
        for c, label in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", "bf16"), ("SQ_INSTS_VALU_MFMA_MOPS_F6F4", "fp4/fp6/fp8")):
            if g(c):
                print(f"- {label} MFMA work: {g(c) * 512 / 1e9:.2f} GFLOP per dispatch ({c} x 512)")
        if g("SQ_LDS_IDX_ACTIVE"):
            print(f"- LDS bank conflicts: {100 * g('SQ_LDS_BANK_CONFLICT', 0.0) / g('SQ_LDS_IDX_ACTIVE'):.2f}% of the "
                  "LDS-active cycles (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE)")
        if g("TCC_EA0_RDREQ") is not None:
            r32, r64, r128 = g("TCC_EA0_RDREQ_32B", 0.0), g("TCC_EA0_RDREQ_64B", 0.0), g("TCC_EA0_RDREQ_128B", 0.0)
            rd = 32 * r32 + 64 * r64 + 128 * r128
            print(f"- reads from memory: {rd / 1e6:.2f} MB per dispatch = 32 x RDREQ_32B + 64 x RDREQ_64B + "
                  f"128 x RDREQ_128B (those three add up to {(r32 + r64 + r128) / max(g('TCC_EA0_RDREQ'), 1):.3f} "
                  "of TCC_EA0_RDREQ)")
            if g("TCC_EA0_RDREQ_DRAM") is not None:
                print(f"- requests served by DRAM: {g('TCC_EA0_RDREQ_DRAM') / max(g('TCC_EA0_RDREQ'), 1):.3f} "
                      "of the read requests (TCC_EA0_RDREQ_DRAM / TCC_EA0_RDREQ)")
        if g("TCC_EA0_WRREQ") is not None:
            w64 = g("TCC_EA0_WRREQ_64B", 0.0)
            wr = 64 * w64 + 32 * (g("TCC_EA0_WRREQ") - w64)
            print(f"- writes to memory: {wr / 1e6:.2f} MB per dispatch = 64 x WRREQ_64B + 32 x (WRREQ - WRREQ_64B)")
            if key == "attention" and g("TCC_EA0_RDREQ") is not None:
                print(f"- attention bytes per launch: {rd + wr:.0f}")
        print()
    return 0


def _time_launches(call, iters: int, warmup: int) -> float:
    """Average microseconds per launch of ``call(i)``, queued behind a spin kernel so
    the events time the kernels back to back rather than the host's submission rate."""
    for i in range(warmup):
        call(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(4_000_000)
    e0.record()
    for i in range(iters):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / iters


def bench_inv_rope_fp8_quant(num_tokens: int, positions, iters: int = 20, warmup: int = 3) -> dict:
    """Event-timed inv_rope_fp8_quant on the attention output (128 heads x 576, rope 64,
    16 groups of 8 heads; two input sets alternated).  Algorithmic bytes: 2 in and 1 out
    per value, 4 per 128-value scale; per token its position and cos/sin row."""
    H, Dh, R, G, P = 128, 576, 64, 16, 65536
    gen = torch.Generator(device="cuda").manual_seed(5)
    sets = [(torch.randn(num_tokens, H, Dh, device="cuda", generator=gen).mul_(0.03).bfloat16(),
             torch.as_tensor(positions if positions is not None else
                             torch.randint(0, P, (num_tokens,), device="cuda", generator=gen),
                             dtype=torch.int32, device="cuda"),
             WL.rope_table(P, R).cuda()) for _ in range(2)]
    D = H // G * Dh
    outs = [(torch.empty((G, num_tokens, D), dtype=torch.uint8, device="cuda"),
             torch.empty((G, num_tokens, D // 128), dtype=torch.float32, device="cuda")) for _ in range(2)]

    def call(i):
        o, pos, cs = sets[i % 2]
        sad.inv_rope_fp8_quant(o, pos, cs, G, out_fp8=outs[i % 2][0], out_scales=outs[i % 2][1])

    us = _time_launches(call, iters, warmup)
    vals = num_tokens * H * Dh
    nbytes = vals * 3 + (vals // 128) * 4 + num_tokens * (4 + 4 * R)
    gbs = nbytes / (us * 1e-6) / 1e9
    del sets, outs
    return {"tokens": num_tokens, "us_per_launch": us, "algorithmic_bytes": nbytes, "achieved_gbs": gbs,
            "hbm_frac": gbs / PEAK_HBM_GBS}


def bench_cache_writes(num_rows: int, iters: int = 30, warmup: int = 3) -> dict:
    """Event-timed insert_kv_rows and insert_index_keys of ``num_rows`` compressed rows into
    pools shaped like the 64K workload's (KV rows 512 fp8 + 64 bf16, pages of 64; indexer
    keys 128 MXFP4), at distinct random slots.  Algorithmic bytes per KV row: 2*576 in,
    672 out, 4 + 4 slot and position, 4*64 cos/sin; per key: 256 in, 68 out, 8, 4*64."""
    g = torch.Generator(device="cuda").manual_seed(9)
    pages = 4096
    kv_pool = torch.zeros((pages, 64 * (640 + 32)), dtype=torch.uint8, device="cuda")
    idx_pool = torch.zeros((pages, 64 * 68), dtype=torch.uint8, device="cuda")
    kv = sad.KvCache(kv_pool, 64, 512, 64)
    idx = sad.IndexerCache(idx_pool, 64, 128)
    rows = torch.randn(num_rows, 576, device="cuda", generator=g).bfloat16()
    keys = torch.randn(num_rows, 128, device="cuda", generator=g).bfloat16()
    pos = torch.randint(0, 65536, (num_rows,), device="cuda", generator=g, dtype=torch.int32)
    slots = torch.randperm(pages * 64, device="cuda", generator=g)[:num_rows].to(torch.int32)
    cs = WL.rope_table(65536, 64).cuda()
    us_kv = _time_launches(lambda i: sad.insert_kv_rows(rows, pos, cs, 4, slots, kv), iters, warmup)
    us_idx = _time_launches(lambda i: sad.insert_index_keys(keys, pos, cs, 4, slots, idx), iters, warmup)
    b_kv = num_rows * (2 * 576 + 672 + 8 + 256)
    b_idx = num_rows * (256 + 68 + 8 + 256)
    del kv_pool, idx_pool
    return {"rows": num_rows,
            "insert_kv_rows": {"us_per_launch": us_kv, "algorithmic_bytes": b_kv,
                               "hbm_frac": b_kv / (us_kv * 1e-6) / 1e9 / PEAK_HBM_GBS},
            "insert_index_keys": {"us_per_launch": us_idx, "algorithmic_bytes": b_idx,
                                  "hbm_frac": b_idx / (us_idx * 1e-6) / 1e9 / PEAK_HBM_GBS}}


def bench_prepare_indexer_q(num_tokens: int, positions, iters: int = 30, warmup: int = 5) -> dict:
    """Event-timed prepare_indexer_q_mxfp4 on 64 heads x 128 dims, rope 64 (two input
    sets alternated).  Algorithmic bytes: per row 2*D in, D/2 + D/32 out, 4 + 4 for the
    weight in and out; per token its position and its cos/sin row (4 + 4*rope)."""
    H, D, R, P = 64, 128, 64, 65536
    sets = [WL.make_indexer_q_inputs(num_tokens, H, D, R, P, seed=31 + i, device="cuda", positions=positions)
            for i in range(2)]
    outs = [(torch.empty((num_tokens, H, D // 2), dtype=torch.uint8, device="cuda"),
             torch.empty((num_tokens, H, D // 32), dtype=torch.uint8, device="cuda"),
             torch.empty((num_tokens, H), dtype=torch.float32, device="cuda")) for _ in range(2)]

    def call(i):
        a, o = sets[i % 2], outs[i % 2]
        sad.prepare_indexer_q_mxfp4(a.index_q, a.positions, a.cos_sin, a.weights, a.softmax_scale,
                                    a.head_scale, q_values=o[0], q_scales=o[1], weights_out=o[2])

    us = _time_launches(call, iters, warmup)
    rows = num_tokens * H
    nbytes = rows * (2 * D + D // 2 + D // 32 + 8) + num_tokens * (4 + 4 * R)
    gbs = nbytes / (us * 1e-6) / 1e9
    del sets, outs
    return {"tokens": num_tokens, "us_per_launch": us, "algorithmic_bytes": nbytes, "achieved_gbs": gbs,
            "hbm_frac": gbs / PEAK_HBM_GBS}


def time_steps(wl: WL.Workload, layers: int, K: int, warmup: int, fused: bool = True):
    """Wall-clock ms per step over K steps (layers rotated) and the mean HIP-event ms of
    the segments: indexer + top-k (from the previous step's end, so launch gaps
    included), index build (0 when fused into the top-k kernel), attention.  The events
    are recorded inside the timed steps, on every EVERY-th step (and the end of the step
    before it), so their cost is spread thin over the timed region."""
    steps = [Step(wl, i) for i in range(layers)]
    for i in range(warmup):
        steps[i % layers].run(fused=fused)
    torch.cuda.synchronize()
    EVERY = 4
    mk = lambda: torch.cuda.Event(enable_timing=True)
    evs = []
    for i in range(K):
        sampled = i % EVERY == 0
        evs.append([mk() if sampled and not fused else None, mk() if sampled else None,
                    mk() if sampled or (i + 1) % EVERY == 0 else None])
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(K):
        steps[i % layers].run(evs[i], fused=fused)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    samples = [i for i in range(0, K, EVERY)]
    attn = [evs[i][1].elapsed_time(evs[i][2]) for i in samples]
    idx = [evs[i - 1][2].elapsed_time(evs[i][0] if not fused else evs[i][1]) for i in samples if i > 0]
    build = [evs[i][0].elapsed_time(evs[i][1]) for i in samples] if not fused else [0.0]
    ms_idx = float(np.mean(idx)) if idx else float("nan")  # needs EVERY + 1 steps
    return wall * 1e3 / K, np.array([ms_idx, np.mean(build), np.mean(attn)])


def time_steps_graph(wl: WL.Workload, layers: int, K: int, warmup: int):
    """Wall-clock ms per step when the steps of all layers are captured once into a HIP
    graph and replayed (every kernel of every step runs on each replay; only the host's
    launch work is replaced).  Before timing, each layer's outputs after a replay are
    checked bit for bit against an eager run of the same step."""
    s = torch.cuda.Stream()
    steps = [Step(wl, i, stream=s) for i in range(layers)]
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for i in range(warmup):
            steps[i % layers].run()
    torch.cuda.synchronize()
    eager = []
    for st in steps:
        with torch.cuda.stream(s):
            st.run()
        torch.cuda.synchronize()
        eager.append((st.topk.clone(), st.si.clone(), st.lens.clone(), st.out.clone()))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for st in steps:
            st.run()
    for st in steps:  # clear the outputs, so the check below sees the replay's writes
        for t in (st.topk, st.si, st.lens, st.out):
            t.zero_()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for st, ref in zip(steps, eager):
        for a, b in zip((st.topk, st.si, st.lens, st.out), ref):
            if not torch.equal(a, b):
                raise RuntimeError("graph replay differs from the eager step")
    reps = max(20, K // layers)
    for _ in range(3):  # the first replays after capture run slower
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del g
    return wall * 1e3 / (reps * layers)


def per_step_ms(wl: WL.Workload, layers: int, n: int, warmup: int, cold: bool = False) -> dict:
    """Per-step HIP-event times of n steps (layers rotated): warm (steps back to back,
    queued behind a spin kernel so the host's launch rate does not show), or cold (a
    1 GiB scratch write, untimed, before each step: the L2s and the 256 MB MALL hold
    none of the step's data).  Median, mean, 10th and 90th percentiles in ms."""
    steps = [Step(wl, i) for i in range(layers)]
    for i in range(warmup):
        steps[i % layers].run()
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    scratch = torch.empty((1 << 28,), dtype=torch.float32, device="cuda") if cold else None
    torch.cuda.synchronize()
    if cold:
        pairs = [(mk(), mk()) for _ in range(n)]
        for i in range(n):
            scratch.fill_(float(i))
            pairs[i][0].record()
            steps[i % layers].run()
            pairs[i][1].record()
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in pairs])
    else:
        ev = [mk() for _ in range(n + 1)]
        torch.cuda._sleep(int(2e5) * n)  # ~0.1 ms of spinning per queued step
        ev[0].record()
        for i in range(n):
            steps[i % layers].run()
            ev[i + 1].record()
        torch.cuda.synchronize()
        ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])
    del scratch
    return {"steps": n, "median_ms": float(np.median(ms)), "mean_ms": float(ms.mean()),
            "p10_ms": float(np.percentile(ms, 10)), "p90_ms": float(np.percentile(ms, 90))}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_rate(wl: WL.Workload, budget_s: float, tokens=None, threads=None) -> dict:
    """The CPU oracle, as it stands, on a bounded sample of tokens of layer 0 (whole step
    each: the indexer, top-k, index build and attention of those tokens); threads: cap the
    BLAS pools (None: as configured)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import sad_oracle as O

    cfg = wl.cfg
    T = wl.num_tokens
    cand = list(range(T)) if tokens is None else list(tokens)

    def run(tok):
        view = WL.host_view(wl, 0, reqs=sorted(set(wl.token_to_req[tok].cpu().tolist())))
        t0 = time.perf_counter()
        O.step(view, cfg, wl.padded_topk, wl.kv_pool.shape[0], wl.idx_pool.shape[0], wl.softmax_scale,
               tokens=tok)
        return time.perf_counter() - t0

    with threadpool_limits(limits=threads):
        t1 = run(cand[:1])
        n = int(max(1, min(len(cand), budget_s / max(t1, 1e-3))))
        tok = cand[:n]
        dt = run(tok) if n > 1 else t1
        used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": n / dt, "unit": "tokens/s", "cores": int(used), "kind": "oracle",
            "sample": f"whole step of {n} of {T} tokens (layer 0), float64 numpy oracle, {dt:.1f} s"
                      + ("" if n == T else "; extrapolated to tokens/s from the sample")}


# The other seeded configurations: (name, layers rotated, oracle sample budget in s)
OTHER_CONFIGS = (("tiny", 1, 3.0), ("b32_8k", 4, 5.0), ("mixed", 1, 8.0), ("dense_1m", 1, 5.0),
                 ("csa_1m", 1, 5.0))


def bench_config(name: str, layers: int, steps: int, warmup: int, oracle_s: float, oracle: bool) -> dict:
    """One seeded configuration: median step time over `steps` per-step events (warm),
    its tokens/s, the attention kernel against both peaks, and the oracle's rate on a
    sample (also single-threaded for the two small configurations)."""
    wl = WL.make_workload(name, "cuda", num_layers=layers)
    torch.cuda.synchronize()
    cfg = wl.cfg
    T = wl.num_tokens
    st = per_step_ms(wl, layers, steps, warmup)
    _, (ms_idx, ms_build, ms_attn) = time_steps(wl, layers, max(steps, 8), warmup)
    ab = algorithmic_bytes(wl)
    gbs = ab["attention"] / (ms_attn * 1e-3) / 1e9
    tf = ab["attention_flops"] / (ms_attn * 1e-3) / 1e12
    res = {"workload": f"{name}: {wl.num_reqs} requests, {T} tokens, max seq {int(wl.seq_lens.max())}, window "
                       f"{cfg.window}, ratio {cfg.ratio}, " + ("dense" if cfg.dense else f"topk {cfg.topk}")
                       + f", {cfg.heads} heads, latent {cfg.d_nope}+{cfg.d_rope}",
           "tokens_per_step": T, "layers_rotated": layers,
           "tokens_per_s": T / (st["median_ms"] * 1e-3), "step": st,
           "kernels_ms": {"indexer_topk_sparse_indices" if not cfg.dense else "build_sparse_indices": ms_idx,
                          "sparse_mla_decode": ms_attn},
           "attention": {"algorithmic_bytes": ab["attention"], "gbs": gbs, "hbm_frac": gbs / PEAK_HBM_GBS,
                         "tflops": tf, "mfma_frac": tf / PEAK_BF16_TFLOPS}}
    if oracle:
        res["cpu_oracle"] = oracle_rate(wl, oracle_s)
        if name in ("tiny", "b32_8k"):
            res["cpu_oracle_single_thread"] = oracle_rate(wl, oracle_s, threads=1)
    del wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def bench_native_record(layers: int, K: int, warmup: int) -> dict:
    """The same 128 x 64K step on the pages' native KV record (448 fp8 + 64 bf16, ue8m0
    scales, 584-byte rows): step rate, and the attention kernel against both peaks."""
    wl = WL.make_workload("b128_64k_native", "cuda", num_layers=layers)
    torch.cuda.synchronize()
    ms_step, (ms_idx, ms_build, ms_attn) = time_steps(wl, layers, K, warmup)
    ab = algorithmic_bytes(wl)
    T = wl.num_tokens
    gbs = ab["attention"] / (ms_attn * 1e-3) / 1e9
    tf = ab["attention_flops"] / (ms_attn * 1e-3) / 1e12
    res = {"workload": "b128_64k_native: as b128_64k, latent 448 fp8 + 64 bf16, ue8m0 scales, "
                       f"kv pool {wl.kv_pool.numel() / 1e9:.1f} GB",
           "tokens_per_s": T / (ms_step * 1e-3), "ms_per_step": ms_step,
           "kernels_ms": {"indexer_topk_sparse_indices": ms_idx, "sparse_mla_decode": ms_attn},
           "attention_algorithmic_bytes": ab["attention"], "attention_gbs": gbs,
           "attention_hbm_frac": gbs / PEAK_HBM_GBS, "attention_tflops": tf,
           "attention_mfma_frac": tf / PEAK_BF16_TFLOPS}
    del wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--layers", type=int, default=4, help="independent layers rotated per step")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--protocol-steps", type=int, default=100,
                    help="per-step median over this many warm and cold steps of the headline")
    ap.add_argument("--no-configs", action="store_true", help="skip the other seeded configurations")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the extra legs (native record, query preparation, output quantization, cache "
                         "writes); counter runs use this so only the step runs")
    ap.add_argument("--summarize-stats", metavar="DIR", help="print a rocprofv3 kernel-stats CSV as markdown")
    ap.add_argument("--summarize-trace", metavar="DIR", help="kernel durations and gaps of a rocprofv3 kernel trace")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="print the step kernels' counters from rocprofv3 --pmc CSV runs")
    args = ap.parse_args()
    if args.summarize_stats:
        return summarize_stats(args.summarize_stats)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters)
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the step is data-parallel "
              "over requests and needs no collectives; run with --gpus 1", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    sad.load()
    t0 = time.perf_counter()
    wl = WL.make_workload(WORKLOAD, "cuda", num_layers=args.layers)
    torch.cuda.synchronize()
    log(f"[bench] workload {WORKLOAD} built in {time.perf_counter() - t0:.1f} s "
        f"(kv pool {wl.kv_pool.numel() / 1e9:.1f} GB, {args.layers} layers)")
    K = args.steps
    # the unfused step first: the first timed configuration of a process runs a few
    # percent slow (first touches of the pools), so it must not be the reported one
    ms_step3, seg3 = time_steps(wl, args.layers, K, args.warmup, fused=False)
    ms_step, (ms_idx, ms_build, ms_attn) = time_steps(wl, args.layers, K, args.warmup)
    ms_graph = time_steps_graph(wl, args.layers, K, args.warmup)
    protocol = {"warm": per_step_ms(wl, args.layers, args.protocol_steps, args.warmup),
                "cold_1gib_scratch_write": per_step_ms(wl, args.layers, args.protocol_steps, args.warmup, cold=True)}
    T = wl.num_tokens
    ab = algorithmic_bytes(wl)
    attn_gbs = ab["attention"] / (ms_attn * 1e-3) / 1e9
    attn_tflops = ab["attention_flops"] / (ms_attn * 1e-3) / 1e12
    idx_gbs = (ab["indexer"] + ab["build"]) / (ms_idx * 1e-3) / 1e9  # the fused indexer + build call
    traffic = measured_traffic()
    cfg = wl.cfg
    result = {
        "metric": "sparse-attn decode tokens/s/GPU at 64K ctx; achieved HBM GB/s % of peak",
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: {wl.num_reqs} requests x 1 decode token, seq_len 65536, "
                               f"window {cfg.window}, compress_ratio {cfg.ratio}, topk {cfg.topk}, "
                               f"{cfg.heads} heads, latent {cfg.d_nope} fp8 + {cfg.d_rope} bf16, indexer "
                               f"{cfg.idx_heads}x{cfg.idx_dim} mxfp4, page {cfg.block}, kv pool "
                               f"{wl.kv_pool.numel() / 1e9:.1f} GB",
                   "tokens_per_step": T, "layers_rotated": args.layers},
        "roofline": {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel": f"sparse_mla_decode ({ATTN_KERNEL})"},
        "roofline_hbm": {"bound": "hbm", "achieved": attn_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": attn_gbs / PEAK_HBM_GBS, "traffic": traffic,
                         "kernel": f"sparse_mla_decode ({ATTN_KERNEL})"},
        "kernels_ms": {"indexer_topk_sparse_indices": ms_idx, "sparse_mla_decode": ms_attn},
        "unfused_step": {"ms_per_step": ms_step3, "tokens_per_s": T / (ms_step3 * 1e-3),
                         "kernels_ms": {"indexer_score_topk": seg3[0], "build_sparse_indices": seg3[1],
                                        "sparse_mla_decode": seg3[2]}},
        "algorithmic_bytes_per_step": {"attention": ab["attention"], "indexer": ab["indexer"],
                                       "build": ab["build"]},
        "graph_replay": {"ms_per_step": ms_graph, "tokens_per_s": T / (ms_graph * 1e-3)},
        "timing_protocol": dict(protocol, cpu_model=cpu_model(),
                                tokens_per_s_warm_median=T / (protocol["warm"]["median_ms"] * 1e-3),
                                tokens_per_s_cold_median=T / (protocol["cold_1gib_scratch_write"]["median_ms"] * 1e-3)),
        "indexer_hbm_gbs": idx_gbs,
        "step_hbm_frac": (ab["attention"] + ab["indexer"] + ab["build"]) / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
        result["cpu_baseline"]["cpu_model"] = cpu_model()
    del wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_configs:
        result["configs"] = {}
        for name, layers, osec in OTHER_CONFIGS:
            log(f"[bench] config {name}")
            result["configs"][name] = bench_config(name, layers, args.protocol_steps, args.warmup, osec,
                                                   not args.no_cpu_baseline)
    if args.no_next_rows:
        print(json.dumps(result), flush=True)
        return 0
    log("[bench] next rows: native KV record, indexer query preparation, output quantization, cache writes")
    native = bench_native_record(args.layers, K, args.warmup)
    result["next_rows"] = {"native_kv_record": native, "prepare_indexer_q_mxfp4": {
        "bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "decode_128_tokens": bench_prepare_indexer_q(T, [65535] * T),
        "prefill_16448_tokens": bench_prepare_indexer_q(16448, None)},
        "inv_rope_fp8_quant": {
        "bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s",
        "decode_128_tokens": bench_inv_rope_fp8_quant(T, [65535] * T),
        "prefill_16448_tokens": bench_inv_rope_fp8_quant(16448, None)},
        "cache_writes": {"bound": "hbm", "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "decode_128_rows": bench_cache_writes(T),
                         "prefill_4112_rows": bench_cache_writes(16448 // 4)}}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
