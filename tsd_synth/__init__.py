"""Seeded synthetic inputs for top-k sparse decode attention.

This module serves both the HIP library's tests/benchmark and the CPU oracle
with the same bytes. It holds none of the method's arithmetic: it only draws
seeded random numbers (torch generators), rounds them to the stored formats
(bf16 / fp16 / OCP FP8 E4M3 via torch's own conversions), shuffles physical
page ids and lays tensors out the way the library takes them.

Workload shapes follow the pages' workloads:
  * double sparsity, "Support double sparsity" (sglang PR #1459), Speedup
    Evaluation: LongChat-7B-shaped (MHA 32/32 heads, FP16, 16 heavy channels,
    1,024 heavy tokens, 20,000-token inputs, batch 3, 200 decode steps) and
    Llama-3.1-8B-shaped (GQA 32/8, 32 heavy channels of K, 3,000 heavy tokens,
    60,000-token inputs, batch 3);
  * QSA-style decode with an FP8 E4M3 cache in 64-token pages ("QSA HiSparse
    -- SGLang plugin", Supported versions) and top_k = 2048 ("HiSparse for
    hybrid DSA/linear-attention models", Speed Tests and Profiling), at 262,144
    tokens per request (8 requests) and at 1,048,576 tokens; and the
    chunked-prefill indexer pass of 2,048 query rows ("Context parallelism for
    QSA attention and the sparse indexer", Motivation; 2,048-token prefill
    chunks in the plugin's Run section).

Distributions: q, K, V, index keys and index queries ~ N(0, 1); index head
weights ~ U(0, 1); double-sparsity K carries a seeded set of outlier channels
per KV head multiplied by a constant before rounding; FP8 pools carry one f32
scale per physical page, amax(page) / 448 (1 for an all-zero page); physical
page ids are a seeded permutation so gathers are non-contiguous.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

PAGE_SIZE = 64
FP8_MAX = 448.0

_TORCH_DTYPE = {"bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass(frozen=True)
class Config:
    """One synthetic workload. ``lens`` overrides ``L`` per request; ``steps``
    > 0 reserves room for that many appended tokens per request (pages are
    allocated for L + steps tokens, lengths start at L + 1)."""
    name: str
    mode: str                    # "ds" (label K) or "qsa" (index K)
    B: int
    L: int
    H_q: int
    H_kv: int
    D: int
    top_k: int
    chunks: int
    kv_enc: str                  # "bf16" | "fp16" | "fp8_e4m3"
    seed: int
    # double sparsity
    r: int = 0
    n_outlier: int = 0
    outlier_scale: float = 1.0
    steps: int = 0
    # QSA index
    H_i: int = 16
    D_i: int = 128
    rows_per_req: int = 1
    prefill_rows: int = 0        # > 0: causal prefill rows at the last positions
    lens: Optional[tuple] = None
    stale_tail: bool = False     # out-of-range page ids past each request's pages
    spare_pages: int = 0
    channel_type: str = "k"      # heavy channels by mean |K|, |q| or |q_c K_c|


WORKLOADS = {
    "ds_tiny_b1_l4096": Config(
        "ds_tiny_b1_l4096", "ds", B=1, L=4096, H_q=8, H_kv=1, D=128,
        top_k=256, chunks=2, kv_enc="bf16", seed=1, r=16, n_outlier=4,
        outlier_scale=8.0),
    "ds_llama7b_b3_l20000_s200": Config(
        "ds_llama7b_b3_l20000_s200", "ds", B=3, L=20000, H_q=32, H_kv=32,
        D=128, top_k=1024, chunks=8, kv_enc="fp16", seed=2, r=16,
        n_outlier=16, outlier_scale=6.0, steps=200),
    "ds_llama31_8b_b3_l60000": Config(
        "ds_llama31_8b_b3_l60000", "ds", B=3, L=60000, H_q=32, H_kv=8, D=128,
        top_k=3000, chunks=24, kv_enc="bf16", seed=3, r=32, n_outlier=32,
        outlier_scale=6.0),
    "qsa_decode_b8_l262144_k2048": Config(
        "qsa_decode_b8_l262144_k2048", "qsa", B=8, L=262144, H_q=32, H_kv=4,
        D=128, top_k=2048, chunks=16, kv_enc="fp8_e4m3", seed=4),
    "qsa_decode_b1_l1048576_k2048": Config(
        "qsa_decode_b1_l1048576_k2048", "qsa", B=1, L=1048576, H_q=32,
        H_kv=4, D=128, top_k=2048, chunks=64, kv_enc="fp8_e4m3", seed=5),
    "qsa_prefill_r2048_l1048576_k2048": Config(
        "qsa_prefill_r2048_l1048576_k2048", "qsa", B=1, L=1048576, H_q=32,
        H_kv=4, D=128, top_k=2048, chunks=64, kv_enc="fp8_e4m3", seed=5,
        prefill_rows=2048),
}


def config(name: str, **overrides) -> Config:
    return replace(WORKLOADS[name], **overrides) if overrides else WORKLOADS[name]


# ------------------------------------------------------------------ helpers
_TAGS = {"pages": 1, "q": 2, "k": 3, "v": 4, "outlier": 5, "index_k": 6,
         "index_q": 7, "index_w": 8, "step_q": 9, "lens": 10}


def _gen(cfg: Config, tag: str, device, layer: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    # the page table (and the index keys of the prefill pass) do not depend on
    # the layer; everything else does
    g.manual_seed((cfg.seed * 1_000_003 + _TAGS[tag] * 7919 + layer * 104_729)
                  % (2**62))
    return g


def _randn(shape, g, device, chunk=1 << 26):
    """N(0,1) float32, drawn in chunks so very large pools stay within
    memory."""
    n = int(np.prod(shape))
    out = torch.empty(n, dtype=torch.float32, device=device)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = torch.randn(e - s, generator=g, device=device)
    return out.view(*shape)


def fp8_codes(x: torch.Tensor) -> torch.Tensor:
    """Round float32 values (|x| <= 448) to OCP FP8 E4M3 codes (uint8) with
    torch's round-to-nearest-even conversion."""
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def quantize_fp8_per_page(x: torch.Tensor, page_size: int = PAGE_SIZE):
    """x: float32 [slots, H, D] -> (codes uint8 [slots, H, D], scale f32
    [slots / page_size]); scale = amax(page) / 448 (1 for an all-zero
    page)."""
    slots = x.shape[0]
    pages = x.reshape(slots // page_size, -1)
    amax = pages.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    codes = torch.empty(pages.shape, dtype=torch.uint8, device=x.device)
    step = max(1, (1 << 26) // max(1, pages.shape[1]))
    for s in range(0, pages.shape[0], step):
        e = min(pages.shape[0], s + step)
        codes[s:e] = fp8_codes(pages[s:e] / scale[s:e, None])
    return codes.view(x.shape), scale.to(torch.float32)


def _lens(cfg: Config):
    if cfg.lens is not None:
        return [int(x) for x in cfg.lens]
    if cfg.steps:
        return [cfg.L + 1] * cfg.B
    return [cfg.L] * cfg.B


def page_layout(cfg: Config, device):
    """(page_table int32 [B, pt_stride], seq_lens int32 [B], num_pages)."""
    lens = _lens(cfg)
    cap_tokens = [max(l, cfg.L + cfg.steps) if cfg.steps else l for l in lens]
    cap = [math.ceil(t / PAGE_SIZE) for t in cap_tokens]
    pt_stride = max(1, max(cap))
    if cfg.stale_tail:
        pt_stride += 3
    num_pages = sum(cap) + cfg.spare_pages
    g = _gen(cfg, "pages", "cpu")
    perm = torch.randperm(max(1, num_pages), generator=g).to(torch.int32)
    pt = torch.zeros((cfg.B, pt_stride), dtype=torch.int32)
    off = 0
    for b in range(cfg.B):
        pt[b, :cap[b]] = perm[off:off + cap[b]]
        off += cap[b]
        if cfg.stale_tail:
            # entries past the request's live pages hold ids no consumer may
            # dereference
            live = math.ceil(lens[b] / PAGE_SIZE)
            tail = pt[b, live:]
            tail.copy_(torch.arange(tail.numel(), dtype=torch.int32) * 7
                       + num_pages + 1000)
            if tail.numel() > 1:
                tail[1::2] = -5
    seq_lens = torch.tensor(lens, dtype=torch.int32)
    return pt.to(device), seq_lens.to(device), num_pages


def _kv_pool(cfg, tag, slots, device, layer, outliers=None):
    x = _randn((slots, cfg.H_kv, cfg.D), _gen(cfg, tag, device, layer), device)
    if outliers is not None:
        # outlier channels of each KV head scaled before rounding
        for g in range(cfg.H_kv):
            x[:, g, outliers[g]] *= cfg.outlier_scale
    if cfg.kv_enc == "fp8_e4m3":
        return quantize_fp8_per_page(x)
    return x.to(_TORCH_DTYPE[cfg.kv_enc]), None


def heavy_channels(k_pool: torch.Tensor, seq_lens, page_table, r: int,
                   prefix_len: int, channel_type: str = "k", q=None):
    """Offline channel choice standing in for calibration ("Support double
    sparsity": heavy channels of type k, q or qk): per KV head, the r
    channels with the largest mean statistic over the first ``prefix_len``
    tokens of every request (ties to the lower channel), listed in ascending
    order. Statistic: |K| (type k); |q| over the group's query heads and the
    requests (type q, from ``q`` [B, H_q, D]); |q_c K_c| with q summed over
    the group (type qk)."""
    H_kv, D = k_pool.shape[1], k_pool.shape[2]
    dev = k_pool.device
    acc = torch.zeros((H_kv, D), dtype=torch.float64, device=dev)
    cnt = 0
    B = page_table.shape[0]
    page_table = page_table.to(dev)
    if channel_type in ("q", "qk"):
        G = q.shape[1] // H_kv
        qg = q.to(dev).to(torch.float64).view(B, H_kv, G, D)
    if channel_type == "q":
        acc = qg.abs().sum(dim=(0, 2))
        cnt = B * G
    else:
        t = torch.arange(prefix_len, device=dev)
        for b in range(B):
            n = min(prefix_len, int(seq_lens[b]))
            tt = t[:n]
            slots = page_table[b, (tt // PAGE_SIZE)].long() * PAGE_SIZE + tt % PAGE_SIZE
            kk = k_pool[slots].to(torch.float64)
            if channel_type == "qk":
                kk = kk * qg[b].sum(dim=1)[None]
            acc += kk.abs().sum(dim=0)
            cnt += n
    mean = acc / max(1, cnt)
    ch = torch.empty((H_kv, r), dtype=torch.int32, device=k_pool.device)
    for g in range(H_kv):
        order = sorted(range(D), key=lambda c: (-float(mean[g, c]), c))[:r]
        ch[g] = torch.tensor(sorted(order), dtype=torch.int32)
    return ch


def make(cfg, device="cpu", layer: int = 0) -> dict:
    """Generate one layer's inputs for ``cfg`` (a Config or a name) on
    ``device``. Returns a dict of torch tensors plus metadata."""
    if isinstance(cfg, str):
        cfg = WORKLOADS[cfg]
    device = torch.device(device)
    pt, seq_lens, num_pages = page_layout(cfg, device)
    slots = num_pages * PAGE_SIZE
    wl = {"cfg": cfg, "mode": cfg.mode, "name": cfg.name, "B": cfg.B,
          "H_q": cfg.H_q, "H_kv": cfg.H_kv, "D": cfg.D, "top_k": cfg.top_k,
          "chunks": cfg.chunks, "page_size": PAGE_SIZE,
          "num_pages": num_pages, "page_table": pt, "seq_lens": seq_lens,
          "kv_enc": cfg.kv_enc}
    q_enc = cfg.kv_enc if cfg.kv_enc in ("bf16", "fp16") else "bf16"
    wl["q_enc"] = q_enc
    qg = _gen(cfg, "q", device, layer)
    wl["q"] = _randn((cfg.B, cfg.H_q, cfg.D), qg, device).to(_TORCH_DTYPE[q_enc])
    if cfg.mode == "ds":
        og = _gen(cfg, "outlier", "cpu", layer)
        outliers = [torch.randperm(cfg.D, generator=og)[:cfg.n_outlier].tolist()
                    for _ in range(cfg.H_kv)]
        wl["outlier_channels"] = outliers
        k_pool, _ = _kv_pool(cfg, "k", slots, device, layer, outliers)
        v_pool, _ = _kv_pool(cfg, "v", slots, device, layer)
        chan = heavy_channels(k_pool, seq_lens.cpu(), pt.cpu(), cfg.r,
                              cfg.L, cfg.channel_type, wl["q"])
        chan = chan.to(device)
        label = torch.gather(
            k_pool, 2,
            chan.long()[None, :, :].expand(slots, cfg.H_kv, cfg.r)).contiguous()
        wl.update(k_pool=k_pool, v_pool=v_pool, k_scale=None, v_scale=None,
                  channel_idx=chan, label_pool=label, r=cfg.r)
        if cfg.steps:
            sg = _gen(cfg, "step_q", device, layer)
            wl["step_q"] = _randn((cfg.steps, cfg.B, cfg.H_q, cfg.D), sg,
                                  device).to(_TORCH_DTYPE[q_enc])
    else:
        k_pool, k_scale = _kv_pool(cfg, "k", slots, device, layer)
        v_pool, v_scale = _kv_pool(cfg, "v", slots, device, layer)
        # index keys belong to the cache, so the prefill pass reads the same
        # keys as the decode workload with the same seed
        ik = _randn((slots, cfg.D_i), _gen(cfg, "index_k", device, layer), device)
        rows = cfg.prefill_rows if cfg.prefill_rows else cfg.B * cfg.rows_per_req
        iq = _randn((rows, cfg.H_i, cfg.D_i),
                    _gen(cfg, "index_q", device, layer), device)
        iw = torch.rand((rows, cfg.H_i), generator=_gen(cfg, "index_w", device,
                                                        layer), device=device)
        wl.update(k_pool=k_pool, v_pool=v_pool, k_scale=k_scale,
                  v_scale=v_scale, index_k=fp8_codes(ik), index_q=fp8_codes(iq),
                  index_w=iw.to(torch.float32), H_i=cfg.H_i, D_i=cfg.D_i)
        if cfg.prefill_rows:
            R = cfg.prefill_rows
            wl["rows_per_req"] = R
            wl["q_pos"] = (torch.arange(R, dtype=torch.int32, device=device)
                           + (int(seq_lens[0]) - R))
        else:
            wl["rows_per_req"] = cfg.rows_per_req
            wl["q_pos"] = None
    return wl


def compressed_layout(wl: dict, block_size: int, seed: int = 0):
    """A paged pool for the block-compressed index keys of a QSA workload:
    ceil(ceil(len / Bs) / 64) compressed pages per request, a seeded
    permutation of physical pages. Returns cpage_table [B, P_c] int32,
    block counts [B] int32, num_cpages and a zeroed pool [cslots, 128]."""
    pt = wl["page_table"]
    dev = pt.device
    B = pt.shape[0]
    nblk = (wl["seq_lens"].to(torch.int64).to(dev) + block_size - 1) // block_size
    cap_blocks = -(-(pt.shape[1] * PAGE_SIZE) // block_size)
    Pc = max(1, -(-cap_blocks // PAGE_SIZE))
    num_cpages = B * Pc
    g = torch.Generator(device="cpu").manual_seed(wl["cfg"].seed * 7919 + seed)
    cpt = torch.randperm(num_cpages, generator=g).view(B, Pc).to(torch.int32)
    pool = torch.zeros((num_cpages * PAGE_SIZE, wl["D_i"]), dtype=torch.uint8,
                       device=dev)
    return {"cpage_table": cpt.to(dev), "block_lens": nblk.to(torch.int32),
            "num_cpages": num_cpages, "ck_pool": pool,
            "block_size": block_size}


def shard_views(wl: dict, W: int):
    """Page-owner shards of a workload's requests (shard w holds the logical
    pages p with p % W == w, in order): per shard, its page table
    [B, ceil(pt_stride / W)] (-1 past its pages) and its token counts [B].
    The pools are shared; only the views differ."""
    pt = wl["page_table"]
    lens = wl["seq_lens"].to(torch.int64).to(pt.device)
    B, P = pt.shape
    Pw = -(-P // W)
    npg = (lens + PAGE_SIZE - 1) // PAGE_SIZE  # logical pages of each row
    last = npg - 1
    tail = lens - last * PAGE_SIZE             # tokens on the last page
    out = []
    for w in range(W):
        cols = torch.arange(w, P, W, device=pt.device)
        ptw = torch.full((B, Pw), -1, dtype=torch.int32, device=pt.device)
        ptw[:, :len(cols)] = pt[:, cols]
        owned = torch.clamp((npg - w + W - 1) // W, min=0)
        lw = owned * PAGE_SIZE
        owns_last = (npg > 0) & (last % W == w)
        lw = torch.where(owns_last, lw - PAGE_SIZE + tail, lw)
        out.append({"page_table": ptw, "seq_lens": lw.to(torch.int32)})
    return out


def to_host(wl: dict) -> dict:
    """Copy a workload to numpy for the CPU oracle: half-precision tensors
    become their uint16 codes, FP8 stays uint8."""
    out = {}
    for k, v in wl.items():
        if isinstance(v, torch.Tensor):
            t = v.detach().cpu()
            if t.dtype in (torch.bfloat16, torch.float16):
                out[k] = t.view(torch.int16).numpy().view(np.uint16)
            else:
                out[k] = t.numpy()
        else:
            out[k] = v
    return out
