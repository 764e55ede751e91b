"""Seeded synthetic workloads for the sparse-attention decode step.

This module only *writes bytes*: it draws N(0,1) data from a seeded torch
generator, encodes it into the two paged cache formats the step reads, lays
the pages out at shuffled physical page ids and builds the ragged batch
descriptors.  It holds none of the step's read-side arithmetic (no decoding,
no scoring, no selection, no index building, no attention), so both the HIP
path and the CPU oracle can consume what it produces without sharing any of
the method's code.

Cache byte layouts (the reader side is defined by the pages' plain-torch
readers: "dequantize_deepseek_v4_fp8_ds_mla_cache" and
"read_deepseek_v4_indexer_mxfp4_cache" on the tokenspeed deepseek_v4_ops page):

* latent KV page (``B`` rows):  ``[B x (Dn e4m3fn bytes | Dr bf16)]`` followed
  by ``[B x Dn/64 fp32 scales]``; one scale per 64-element block,
  ``scale = max(amax, 1e-4) / 448`` (fp32), ``byte = e4m3_rne(clamp(x/scale, +-448))``.
* indexer key page (``Bi`` rows): ``[Bi x Di/2]`` packed E2M1 (low nibble =
  even element) followed by ``[Bi x Di/32]`` e8m0 exponents (``2^(b-127)``).
  Encoder: ``e = ceil(log2(amax/6))`` per 32-element block, element
  ``= e2m1_rne_saturating(x / 2^e)``.

Every workload is deterministic for a given (config, device): data is drawn
from one ``torch.Generator`` seeded with the config seed, in a fixed order.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

FP8_MAX = 448.0
FP8_BLOCK = 64
MX_BLOCK = 32
E2M1_MAX = 6.0


# --------------------------------------------------------------------------
# Workload shapes
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class Config:
    """One workload shape (batch geometry, head/latent dims, cache formats)."""

    name: str
    seed: int
    window: int
    ratio: int
    topk: int  # 0 = dense compressed path (no indexer)
    heads: int
    d_nope: int
    d_rope: int
    idx_heads: int
    idx_dim: int
    block: int  # KV page rows
    idx_block: int  # indexer page rows
    # batch description: list of (num_reqs, q_len, seq_len or (lo, hi), replay) groups
    groups: tuple = ()
    kv_pool_pages: int = 0  # 0 = 4x the used pages
    idx_pool_pages: int = 0
    swa_backing: str = "window"  # "window" | "all"
    pin_first_prefill_seq: int = 0  # config 4 pins one prefill request's seq len
    kv_format: str = "f32"  # "f32": fp32 scale per 64 nope values; "ue8m0": the pages' native record
    # 0: window rows share the compressed rows' pool and page size; else the window rows
    # live in a pool of their own with this many rows per page (two caches, as the
    # attention backend keeps them)
    swa_block: int = 0
    swa_pool_pages: int = 0  # 0 = 4x the window pages used (two-cache form only)

    @property
    def dqk(self) -> int:
        return self.d_nope + self.d_rope

    @property
    def dense(self) -> bool:
        return self.topk == 0

    @property
    def kv_row_bytes(self) -> int:
        return self.d_nope + 2 * self.d_rope

    @property
    def kv_scale_bytes(self) -> int:
        # native record: one ue8m0 byte per 64 nope values, padded to 8 bytes per row
        return 8 if self.kv_format == "ue8m0" else 4 * (self.d_nope // FP8_BLOCK)

    @property
    def kv_page_bytes(self) -> int:
        return self.block * (self.kv_row_bytes + self.kv_scale_bytes)

    @property
    def two_cache(self) -> bool:
        return self.swa_block != 0

    @property
    def swa_block_size(self) -> int:
        return self.swa_block or self.block

    @property
    def swa_page_bytes(self) -> int:
        return self.swa_block_size * (self.kv_row_bytes + self.kv_scale_bytes)

    @property
    def idx_row_bytes(self) -> int:
        return self.idx_dim // 2

    @property
    def idx_scale_bytes(self) -> int:
        return self.idx_dim // MX_BLOCK

    @property
    def idx_page_bytes(self) -> int:
        return self.idx_block * (self.idx_row_bytes + self.idx_scale_bytes)


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


CONFIGS = {
    # 1 request, 1 decode token at seq 256, W=32, ratio 4 (64 compressed rows), k=16
    "tiny": Config(
        name="tiny", seed=0, window=32, ratio=4, topk=16, heads=8, d_nope=128, d_rope=32,
        idx_heads=4, idx_dim=64, block=16, idx_block=16,
        groups=((1, 1, 256, 0),), kv_pool_pages=64, idx_pool_pages=8, swa_backing="all",
    ),
    # 32 requests x 1 token, seq 8192, W=128, ratio 4 (2048 rows), k=512, 64 heads
    "b32_8k": Config(
        name="b32_8k", seed=1, window=128, ratio=4, topk=512, heads=64, d_nope=512, d_rope=64,
        idx_heads=64, idx_dim=128, block=64, idx_block=64, groups=((32, 1, 8192, 0),),
    ),
    # 128 requests x 1 token, seq 65536, W=128, ratio 4 (16384 rows), k=2048, 128 heads,
    # pages shuffled over a ~196 GB KV pool and a ~3.9 GB indexer pool
    "b128_64k": Config(
        name="b128_64k", seed=2, window=128, ratio=4, topk=2048, heads=128, d_nope=512,
        d_rope=64, idx_heads=64, idx_dim=128, block=64, idx_block=64,
        groups=((128, 1, 65536, 0),), kv_pool_pages=4_560_000, idx_pool_pages=900_000,
    ),
    # 64 decode tokens at seq 16384 first, then 4 prefill chunks of 4096 tokens with
    # seq ~ U[4096, 32768] (first pinned to 4096) and replay_start ~ U[0, seq/2]
    "mixed": Config(
        name="mixed", seed=3, window=128, ratio=4, topk=2048, heads=128, d_nope=512,
        d_rope=64, idx_heads=64, idx_dim=128, block=64, idx_block=64,
        groups=((64, 1, 16384, 0), (4, 4096, (4096, 32768), "half")),
        pin_first_prefill_seq=4096,
    ),
    # the pages' native KV record (448 fp8 + 64 bf16, ue8m0 scales): small and 64K shapes
    "tiny_native": Config(
        name="tiny_native", seed=10, window=32, ratio=4, topk=16, heads=8, d_nope=448, d_rope=64,
        idx_heads=4, idx_dim=64, block=16, idx_block=16,
        groups=((1, 1, 256, 0),), kv_pool_pages=64, idx_pool_pages=8, swa_backing="all",
        kv_format="ue8m0",
    ),
    "b32_8k_native": Config(
        name="b32_8k_native", seed=11, window=128, ratio=4, topk=512, heads=64, d_nope=448, d_rope=64,
        idx_heads=64, idx_dim=128, block=64, idx_block=64, groups=((32, 1, 8192, 0),),
        kv_format="ue8m0",
    ),
    "b128_64k_native": Config(
        name="b128_64k_native", seed=12, window=128, ratio=4, topk=2048, heads=128, d_nope=448,
        d_rope=64, idx_heads=64, idx_dim=128, block=64, idx_block=64,
        groups=((128, 1, 65536, 0),), kv_pool_pages=4_560_000, idx_pool_pages=900_000,
        kv_format="ue8m0",
    ),
    # two caches (the attention backend's window cache and compressed cache, each with its
    # own pool and page size): window pages of 64 rows, compressed pages of 16 rows
    "two_cache_tiny": Config(
        name="two_cache_tiny", seed=20, window=32, ratio=4, topk=16, heads=8, d_nope=128, d_rope=32,
        idx_heads=4, idx_dim=64, block=16, idx_block=16, groups=((1, 1, 256, 0), (1, 40, 300, 12)),
        swa_backing="all", swa_block=64,
    ),
    "two_cache_b8_8k": Config(
        name="two_cache_b8_8k", seed=21, window=128, ratio=4, topk=512, heads=64, d_nope=512,
        d_rope=64, idx_heads=64, idx_dim=128, block=16, idx_block=64, groups=((8, 1, 8192, 0),),
        swa_block=64,
    ),
    # 8 requests at seq 1M, ratio 128 (8192 compressed rows, all attended), W=128
    # 4 requests x 1 token at seq 2^20, ratio 4: 262144 compressed rows, past one top-k
    # workgroup's reach (8 chunks of 32768 rows, merged)
    "csa_1m": Config(
        name="csa_1m", seed=22, window=128, ratio=4, topk=2048, heads=128, d_nope=512,
        d_rope=64, idx_heads=64, idx_dim=128, block=64, idx_block=64,
        groups=((4, 1, 1 << 20, 0),),
    ),
    "dense_1m": Config(
        name="dense_1m", seed=4, window=128, ratio=128, topk=0, heads=128, d_nope=512,
        d_rope=64, idx_heads=64, idx_dim=128, block=64, idx_block=64,
        groups=((8, 1, 1 << 20, 0),), kv_pool_pages=4_560_000,
    ),
}

# The headline workload (128 requests at 64K context).
HEADLINE = "b128_64k"


def kv_scale_format(cfg: Config) -> int:
    """The C ABI's scale_format of the config's KV cache (0: fp32 scales, 1: ue8m0 bytes)."""
    return 1 if cfg.kv_format == "ue8m0" else 0


def padded_topk(cfg: Config, max_seq: int) -> int:
    """Width of the compressed segment: max(k, widest dense row) rounded to 64."""
    widest = max_seq // cfg.ratio if cfg.dense else cfg.topk
    return _round_up(max(widest, 1), 64)


# --------------------------------------------------------------------------
# Encoders (write side only)
# --------------------------------------------------------------------------


def encode_fp8_rows(x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """bf16-valued rows [N, Dn] -> (e4m3fn bytes [N, Dn], fp32 scales [N, Dn/64])."""
    n, dn = x.shape
    blocks = x.float().reshape(n, dn // FP8_BLOCK, FP8_BLOCK)
    amax = blocks.abs().amax(dim=-1).clamp_min(1.0e-4)
    scale = amax / FP8_MAX  # fp32 division
    y = torch.clamp(blocks / scale.unsqueeze(-1), -FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, dn)
    return codes, scale.contiguous()


def encode_fp8_rows_ue8m0(x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """bf16-valued rows [N, Dn] -> (e4m3fn bytes [N, Dn], ue8m0 scale bytes [N, 8]): the
    pages' native writer rule, exponent = ceil(log2(max(amax, 1e-4) / 448)) per 64 values,
    values x * 2^-exponent, byte = exponent + 127, padded with zeros to 8 bytes."""
    n, dn = x.shape
    blocks = x.float().reshape(n, dn // FP8_BLOCK, FP8_BLOCK)
    amax = blocks.abs().amax(dim=-1).clamp_min(1.0e-4)
    exponent = torch.ceil(torch.log2(amax / FP8_MAX))
    y = torch.clamp(blocks * torch.pow(2.0, -exponent).unsqueeze(-1), -FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, dn)
    sb = torch.zeros((n, 8), dtype=torch.uint8, device=x.device)
    sb[:, : dn // FP8_BLOCK] = torch.clamp(exponent + 127.0, 0.0, 255.0).to(torch.uint8)
    return codes, sb.contiguous()


# Round-to-nearest-even thresholds on the E2M1 magnitude grid
# {0, .5, 1, 1.5, 2, 3, 4, 6}: the code is the count of thresholds passed; a
# midpoint goes to the even code (strict ">" where the lower code is even).
_E2M1_UP = ((0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False),
            (3.5, True), (5.0, False))


def encode_mxfp4(x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """fp32 vectors [N, D] -> (packed nibbles [N, D/2] u8, e8m0 exponents [N, D/32] u8)."""
    n, d = x.shape
    blocks = x.float().reshape(n, d // MX_BLOCK, MX_BLOCK)
    amax = blocks.abs().amax(dim=-1).clamp_min(1.0e-30)
    e = torch.ceil(torch.log2(amax / E2M1_MAX)).clamp(-127, 127)
    y = blocks / torch.pow(2.0, e).unsqueeze(-1)
    mag = y.abs()
    code = torch.zeros_like(mag, dtype=torch.int32)
    for thr, inclusive in _E2M1_UP:
        code += (mag >= thr).int() if inclusive else (mag > thr).int()
    code = code.clamp(max=7)
    code = code | ((y < 0).int() << 3)
    code = code.reshape(n, d).to(torch.uint8)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), (e + 127).to(torch.uint8).contiguous()


def _bf16_round(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


# --------------------------------------------------------------------------
# Workload construction
# --------------------------------------------------------------------------


@dataclass
class Layer:
    """Per-layer inputs: tables, queries and indexer inputs."""

    swa_bt: torch.Tensor  # [R, swa_cols] int32
    comp_bt: torch.Tensor  # [R, comp_cols] int32
    idx_bt: torch.Tensor  # [R, idx_cols] int32 (dense: [R, 1] of -1)
    q: torch.Tensor  # [T, H, Dqk] bf16
    idx_q_values: torch.Tensor  # [T, Hi, Di/2] u8
    idx_q_scales: torch.Tensor  # [T, Hi, Di/32] u8
    idx_weights: torch.Tensor  # [T, Hi] fp32, pre-folded
    kv_pages: list = field(default_factory=list)  # physical KV pages written
    idx_pages: list = field(default_factory=list)


@dataclass
class Workload:
    cfg: Config
    device: torch.device
    num_reqs: int
    num_tokens: int
    query_start_loc: torch.Tensor  # [R+1] int32
    seq_lens: torch.Tensor  # [R] int32
    token_to_req: torch.Tensor  # [T] int32
    replay_start: torch.Tensor  # [R] int32
    padded_topk: int
    softmax_scale: float
    kv_pool: torch.Tensor  # [pages, page_bytes] u8 (compressed rows; window rows too unless two-cache)
    idx_pool: torch.Tensor  # [pages, idx_page_bytes] u8 (1 page when dense)
    layers: list
    swa_pool: torch.Tensor = None  # window rows' pool: kv_pool itself unless cfg.two_cache

    @property
    def max_seq(self) -> int:
        return int(self.seq_lens.max().item()) if self.num_reqs else 0


def _geometry(cfg: Config, gen: torch.Generator):
    q_lens, seq_lens, replay = [], [], []
    first_prefill = True
    for nreq, qlen, seq, rep in cfg.groups:
        for _ in range(nreq):
            if isinstance(seq, tuple):
                lo, hi = seq
                s = int(torch.randint(lo, hi + 1, (1,), generator=gen).item())
                if first_prefill and cfg.pin_first_prefill_seq:
                    s = cfg.pin_first_prefill_seq
                first_prefill = False
            else:
                s = seq
            if rep == "half":
                r = int(torch.randint(0, s // 2 + 1, (1,), generator=gen).item())
            else:
                r = int(rep)
            q_lens.append(qlen)
            seq_lens.append(s)
            replay.append(r)
    return q_lens, seq_lens, replay


def _kv_page_bytes(cfg: Config, rows: torch.Tensor, B: int = 0) -> torch.Tensor:
    """Encode rows [npages*B, Dqk] (bf16) into page images [npages, page_bytes]."""
    B = B or cfg.block
    n = rows.shape[0]
    npages = n // B
    nope = rows[:, : cfg.d_nope]
    rope = rows[:, cfg.d_nope:].contiguous()
    if cfg.kv_format == "ue8m0":
        codes, scales = encode_fp8_rows_ue8m0(nope.float())
    else:
        codes, scales = encode_fp8_rows(nope.float())
    vals = torch.cat([codes, rope.view(torch.uint8).reshape(n, 2 * cfg.d_rope)], dim=1)
    vals = vals.reshape(npages, B * cfg.kv_row_bytes)
    sc = scales.view(torch.uint8).reshape(npages, B * cfg.kv_scale_bytes)
    return torch.cat([vals, sc], dim=1)


def _idx_page_bytes(cfg: Config, keys: torch.Tensor) -> torch.Tensor:
    Bi = cfg.idx_block
    n = keys.shape[0]
    npages = n // Bi
    packed, exps = encode_mxfp4(keys)
    return torch.cat(
        [packed.reshape(npages, Bi * cfg.idx_row_bytes), exps.reshape(npages, Bi * cfg.idx_scale_bytes)],
        dim=1,
    )


def make_workload(
    cfg: Config | str,
    device: str | torch.device = "cpu",
    *,
    num_layers: int = 1,
    kv_pool_pages: int | None = None,
    idx_pool_pages: int | None = None,
    q_scale: float = 1.0,
) -> Workload:
    """Build a seeded workload.

    ``q_scale`` multiplies the attention queries (the "peaky" variant uses 4);
    pool sizes default to the config's (or 4x the pages actually used).
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    device = torch.device(device)
    gen = torch.Generator(device="cpu")
    gen.manual_seed(cfg.seed)
    q_lens, seq_lens, replay = _geometry(cfg, gen)
    R = len(q_lens)
    T = sum(q_lens)
    qsl = [0]
    for ql in q_lens:
        qsl.append(qsl[-1] + ql)
    token_to_req = [r for r in range(R) for _ in range(q_lens[r])]
    max_seq = max(seq_lens)
    P = padded_topk(cfg, max_seq)
    B, Bi, W = cfg.block, cfg.idx_block, cfg.window
    Bs = cfg.swa_block_size

    # Which logical pages each request needs.
    n_comp = [s // cfg.ratio for s in seq_lens]
    comp_pages = [(nc + B - 1) // B for nc in n_comp]
    idx_pages = [0 if cfg.dense else (nc + Bi - 1) // Bi for nc in n_comp]
    swa_cols = (max_seq + Bs - 1) // Bs
    swa_needed = []
    for r in range(R):
        first_pos = seq_lens[r] - q_lens[r]
        lo = max(first_pos - W + 1, replay[r], 0)
        if cfg.swa_backing == "all":
            lo = 0
        lo_page = lo // Bs
        hi_page = (seq_lens[r] - 1) // Bs
        swa_needed.append(list(range(lo_page, hi_page + 1)) if lo <= seq_lens[r] - 1 else [])
    swa_used = sum(len(x) for x in swa_needed)
    kv_used = sum(comp_pages) + (0 if cfg.two_cache else swa_used)
    idx_used = sum(idx_pages)
    n_kv_pages = kv_pool_pages or cfg.kv_pool_pages or 4 * kv_used * num_layers
    n_idx_pages = idx_pool_pages or cfg.idx_pool_pages or max(1, 4 * idx_used * num_layers)
    n_swa_pages = (cfg.swa_pool_pages or max(1, 4 * swa_used * num_layers)) if cfg.two_cache else 0
    if (kv_used * num_layers > n_kv_pages or idx_used * num_layers > n_idx_pages
            or (cfg.two_cache and swa_used * num_layers > n_swa_pages)):
        raise ValueError("pool too small for the requested layers")
    if n_kv_pages * B >= 2**31 or n_idx_pages * Bi >= 2**31 or n_swa_pages * Bs >= 2**31:
        raise ValueError("slot ids must fit int32")

    # Device-side generator for the bulk data.
    dgen = torch.Generator(device=device)
    dgen.manual_seed(cfg.seed * 1000 + 17)

    kv_pool = torch.empty((n_kv_pages, cfg.kv_page_bytes), dtype=torch.uint8, device=device)
    idx_pool = torch.empty((n_idx_pages, cfg.idx_page_bytes), dtype=torch.uint8, device=device)
    kv_perm = torch.randperm(n_kv_pages, generator=dgen, device=device)[: kv_used * num_layers]
    idx_perm = torch.randperm(n_idx_pages, generator=dgen, device=device)[: idx_used * num_layers]
    kv_perm_l = kv_perm.cpu().tolist()
    idx_perm_l = idx_perm.cpu().tolist()
    kv_next = 0
    idx_next = 0
    if cfg.two_cache:
        swa_pool = torch.empty((n_swa_pages, cfg.swa_page_bytes), dtype=torch.uint8, device=device)
        swa_perm_l = torch.randperm(n_swa_pages, generator=dgen, device=device)[: swa_used * num_layers].cpu().tolist()
        swa_next = 0
    else:
        swa_pool = kv_pool

    comp_cols = max(1, max(comp_pages))
    idx_cols = max(1, max(idx_pages))
    layers = []
    for layer in range(num_layers):
        swa_bt = torch.full((R, swa_cols), -1, dtype=torch.int32)
        comp_bt = torch.full((R, comp_cols), -1, dtype=torch.int32)
        idx_bt = torch.full((R, idx_cols), -1, dtype=torch.int32)
        kv_written = []
        idx_written = []
        for r in range(R):
            # compressed rows: one latent row per compressed position
            pages = kv_perm_l[kv_next: kv_next + comp_pages[r]]
            kv_next += comp_pages[r]
            comp_bt[r, : len(pages)] = torch.tensor(pages, dtype=torch.int32)
            if pages:
                rows = _bf16_round(torch.randn((len(pages) * B, cfg.dqk), generator=dgen, device=device))
                kv_pool[torch.tensor(pages, device=device)] = _kv_page_bytes(cfg, rows)
                kv_written += pages
            # window rows: one latent row per token position
            if cfg.two_cache:
                spages = swa_perm_l[swa_next: swa_next + len(swa_needed[r])]
                swa_next += len(swa_needed[r])
            else:
                spages = kv_perm_l[kv_next: kv_next + len(swa_needed[r])]
                kv_next += len(swa_needed[r])
            for lp, pp in zip(swa_needed[r], spages):
                swa_bt[r, lp] = pp
            if spages:
                rows = _bf16_round(torch.randn((len(spages) * Bs, cfg.dqk), generator=dgen, device=device))
                swa_pool[torch.tensor(spages, device=device)] = _kv_page_bytes(cfg, rows, Bs)
                if not cfg.two_cache:
                    kv_written += spages
            # indexer keys (MXFP4), one per compressed row
            if not cfg.dense:
                ipages = idx_perm_l[idx_next: idx_next + idx_pages[r]]
                idx_next += idx_pages[r]
                idx_bt[r, : len(ipages)] = torch.tensor(ipages, dtype=torch.int32)
                if ipages:
                    keys = torch.randn((len(ipages) * Bi, cfg.idx_dim), generator=dgen, device=device)
                    idx_pool[torch.tensor(ipages, device=device)] = _idx_page_bytes(cfg, keys)
                    idx_written += ipages
        q = _bf16_round(
            torch.randn((T, cfg.heads, cfg.dqk), generator=dgen, device=device) * q_scale
        )
        if cfg.dense:
            iqv = torch.zeros((T, cfg.idx_heads, cfg.idx_dim // 2), dtype=torch.uint8, device=device)
            iqs = torch.full((T, cfg.idx_heads, cfg.idx_dim // MX_BLOCK), 127, dtype=torch.uint8, device=device)
            iw = torch.zeros((T, cfg.idx_heads), dtype=torch.float32, device=device)
        else:
            iq = torch.randn((T * cfg.idx_heads, cfg.idx_dim), generator=dgen, device=device)
            iqv, iqs = encode_mxfp4(iq)
            iqv = iqv.reshape(T, cfg.idx_heads, cfg.idx_dim // 2)
            iqs = iqs.reshape(T, cfg.idx_heads, cfg.idx_dim // MX_BLOCK)
            # weights pre-folded with softmax_scale = Di^-1/2 and head_scale = Hi^-1/2
            iw = (
                torch.randn((T, cfg.idx_heads), generator=dgen, device=device)
                * (cfg.idx_dim ** -0.5) * (cfg.idx_heads ** -0.5)
            ).float()
        layers.append(
            Layer(
                swa_bt=swa_bt.to(device), comp_bt=comp_bt.to(device), idx_bt=idx_bt.to(device),
                q=q.contiguous(), idx_q_values=iqv.contiguous(), idx_q_scales=iqs.contiguous(),
                idx_weights=iw.contiguous(), kv_pages=kv_written, idx_pages=idx_written,
            )
        )

    i32 = dict(dtype=torch.int32, device=device)
    return Workload(
        cfg=cfg,
        device=device,
        num_reqs=R,
        num_tokens=T,
        query_start_loc=torch.tensor(qsl, **i32),
        seq_lens=torch.tensor(seq_lens, **i32),
        token_to_req=torch.tensor(token_to_req, **i32),
        replay_start=torch.tensor(replay, **i32),
        padded_topk=P,
        softmax_scale=cfg.dqk ** -0.5,
        kv_pool=kv_pool,
        idx_pool=idx_pool,
        layers=layers,
        swa_pool=swa_pool,
    )


# --------------------------------------------------------------------------
# Host views (data movement only) for the CPU oracle
# --------------------------------------------------------------------------


@dataclass
class HostView:
    """numpy copies of one layer's inputs; pools as {physical page: bytes}."""

    query_start_loc: object
    seq_lens: object
    token_to_req: object
    replay_start: object
    swa_bt: object
    comp_bt: object
    idx_bt: object
    q: object  # [T, H, Dqk] uint16 bf16 bits
    idx_q_values: object
    idx_q_scales: object
    idx_weights: object
    kv_pages: dict  # pages of the compressed rows' pool (and of the window rows' unless two-cache)
    idx_pages: dict
    swa_pages: dict = None  # pages of the window rows' pool (kv_pages itself unless two-cache)


def _copy_pages(pool: torch.Tensor, ids, device) -> dict:
    pages = {}
    chunk = 4096
    for i in range(0, len(ids), chunk):
        part = ids[i: i + chunk]
        data = pool[torch.tensor(part, device=device)].detach().cpu().numpy()
        for j, pid in enumerate(part):
            pages[pid] = data[j]
    return pages


def host_view(wl: Workload, layer: int = 0, reqs=None) -> HostView:
    """Copy one layer to host numpy arrays.

    Only the pages referenced by the block tables of ``reqs`` (default: every
    request) are copied; the pools may be far larger than host memory.
    """
    L = wl.layers[layer]

    def np_(t):
        return t.detach().cpu().numpy()

    rows = slice(None) if reqs is None else torch.as_tensor(sorted(set(reqs)), device=L.swa_bt.device)

    def ids_in(tables, pool):
        # only ids that name a page of the pool (tables may hold -1 or stale ids past it)
        ids = torch.cat([t[rows].flatten() for t in tables])
        return sorted(set(ids[(ids >= 0) & (ids < pool.shape[0])].cpu().tolist()))

    two = wl.swa_pool is not None and wl.swa_pool is not wl.kv_pool
    kv_tables = [L.comp_bt] if two else [L.swa_bt, L.comp_bt]
    kv_pages = _copy_pages(wl.kv_pool, ids_in(kv_tables, wl.kv_pool), wl.device)
    idx_pages = _copy_pages(wl.idx_pool, ids_in([L.idx_bt], wl.idx_pool), wl.device)
    swa_pages = _copy_pages(wl.swa_pool, ids_in([L.swa_bt], wl.swa_pool), wl.device) if two else kv_pages
    return HostView(
        query_start_loc=np_(wl.query_start_loc),
        seq_lens=np_(wl.seq_lens),
        token_to_req=np_(wl.token_to_req),
        replay_start=np_(wl.replay_start),
        swa_bt=np_(L.swa_bt),
        comp_bt=np_(L.comp_bt),
        idx_bt=np_(L.idx_bt),
        q=np_(L.q.view(torch.int16)).view("uint16"),
        idx_q_values=np_(L.idx_q_values),
        idx_q_scales=np_(L.idx_q_scales),
        idx_weights=np_(L.idx_weights),
        kv_pages=kv_pages,
        idx_pages=idx_pages,
        swa_pages=swa_pages,
    )


def with_overrides(cfg: Config, **kw) -> Config:
    """A variant of a config (e.g. the sparse-equals-dense self-check)."""
    return replace(cfg, **kw)


# --------------------------------------------------------------------------
# Inputs of the indexer query preparation (RoPE, Hadamard, MXFP4, weight fold)
# --------------------------------------------------------------------------


@dataclass
class IndexerQInputs:
    index_q: torch.Tensor  # [T, Hi, Di] bf16, N(0, 1)
    positions: torch.Tensor  # [T] int32
    cos_sin: torch.Tensor  # [max_pos, rope_dim] fp32: cos columns, then sin
    weights: torch.Tensor  # [T, Hi] fp32, N(0, 1), before the fold
    softmax_scale: float  # Di^-1/2
    head_scale: float  # Hi^-1/2


def rope_table(max_pos: int, rope_dim: int, base: float = 10000.0) -> torch.Tensor:
    """Rotary cos/sin table [max_pos, rope_dim] fp32: angle(p, i) = p * base^(-2i/rope_dim)."""
    inv = base ** (-torch.arange(rope_dim // 2, dtype=torch.float64) * 2.0 / rope_dim)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * inv[None, :]
    return torch.cat([torch.cos(ang), torch.sin(ang)], dim=1).float().contiguous()


def make_indexer_q_inputs(num_tokens: int, idx_heads: int, idx_dim: int, rope_dim: int, max_pos: int,
                          seed: int, device="cpu", positions=None) -> IndexerQInputs:
    """Seeded inputs; positions are uniform in [0, max_pos) unless given."""
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(num_tokens, idx_heads, idx_dim, generator=g).bfloat16()
    w = torch.randn(num_tokens, idx_heads, generator=g)
    if positions is None:
        positions = torch.randint(0, max_pos, (num_tokens,), generator=g)
    positions = torch.as_tensor(positions, dtype=torch.int32)
    return IndexerQInputs(q.to(device), positions.to(device), rope_table(max_pos, rope_dim).to(device),
                          w.to(device), idx_dim ** -0.5, idx_heads ** -0.5)
