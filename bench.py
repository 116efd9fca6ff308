"""Benchmark of one sparse-decode step on one MI355X.

A step is the whole path over one batch: sparse_index_score -> topk_select
-> sparse_gqa_decode -> lse_merge, on one layer's inputs. Steps rotate over
``--replicas`` layers with their own pools so the bytes scanned between two
visits of the same layer exceed the 256 MB Infinity Cache. Inputs are seeded
synthetic tensors already resident in HBM when the timed region starts.

Prints one JSON line: steps/s (whole-job throughput), the model HBM rate of
the step, the roofline of the dominant kernel (the index-K scan) from HIP
events on the launch stream, and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = ("sparse-decode steps/s + achieved HBM GB/s (% roofline) at 262K ctx, "
          "top_k=2048")


def model_bytes(cfg):
    """Algorithmic bytes of one step: the index (or label) keys of every
    cached token plus the K and V rows of the selected tokens."""
    B, L, k = cfg.B, (cfg.lens[0] if cfg.lens else cfg.L), cfg.top_k
    kv_b = 1 if cfg.kv_enc == "fp8_e4m3" else 2
    if cfg.mode == "qsa":
        index = B * L * cfg.D_i                      # FP8 index key per token
        gather = B * k * cfg.H_kv * cfg.D * 2 * kv_b  # shared selection
    else:
        index = B * L * cfg.H_kv * cfg.r * kv_b      # label per token and head
        gather = B * cfg.H_kv * k * cfg.D * 2 * kv_b  # per-head selection
    return index, gather


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(layer, seconds):
    """The CPU oracle as it stands (plain C, double accumulation) on whole
    requests of one decode step, about ``seconds`` of CPU work in all: first
    one thread, request after request (cycling over the step's requests),
    for two thirds of it; then every usable core, one request per task, for
    about ``seconds`` more CPU-seconds (at least one task per core and one
    step's worth; the oracle's calls release the interpreter lock, so the
    threads run in parallel). Both scaled to steps/s (requests done /
    requests per step / wall time)."""
    import concurrent.futures as cf

    import oracle
    import tsd_synth
    h = tsd_synth.to_host(layer)
    B = h["B"]

    def one(b):
        sub = dict(h)
        sub["B"] = 1
        for key in ("q", "page_table", "seq_lens"):
            sub[key] = h[key][b:b + 1]
        if h["mode"] == "qsa":
            sub["index_q"] = h["index_q"][b:b + 1]
            sub["index_w"] = h["index_w"][b:b + 1]
        oracle.decode_step(sub)

    oracle._load()
    done, t0 = 0, time.perf_counter()
    while True:
        one(done % B)
        done += 1
        if time.perf_counter() - t0 >= seconds * 2 / 3:
            break
    el1 = time.perf_counter() - t0
    single = (done / B) / el1
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    per_request = el1 / done
    tasks = max(B, cores, math.ceil(seconds / per_request))
    tasks = (tasks + cores - 1) // cores * cores
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        list(ex.map(one, [i % B for i in range(tasks)]))
    elN = time.perf_counter() - t0
    what = (f"every cached token scored, exact top-{h['top_k']}, sparse "
            f"attention over {h['H_q']} heads, merge")
    return {"value": (tasks / B) / elN, "unit": "steps/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{tasks} request-tasks ({B} requests per step; each: "
                      f"{what}) on {cores} threads in {elN:.1f} s; one "
                      f"thread: {done} requests in {el1:.1f} s; "
                      f"scaled to steps/s",
            "single_thread": {"value": single, "unit": "steps/s", "cores": 1},
            "nproc": os.cpu_count(), "cpu_model": _cpu_model()}


TRAFFIC_RECORD = os.path.join(ROOT, "profiles",
                              "qsa_decode_b8_l262144_k2048.hbm_traffic.md")
SCAN_SOURCES = ("score_qsa.hip", "device_common.h", "topk_common.h")


def scan_traffic():
    """HBM bytes per launch of the index scan from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when the
    scan's sources have changed since those counters were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_RECORD).read()
    except OSError:
        return None
    rec = dict(line.strip().split(": ", 1) for line in text.splitlines()
               if line.strip().startswith(("scan_traffic_bytes_per_launch:",
                                           "scan_sources_sha256:")))
    h = hashlib.sha256()
    for name in SCAN_SOURCES:
        with open(os.path.join(ROOT, "top_sparse_decode_amd", "csrc", name),
                  "rb") as f:
            h.update(f.read())
    if rec.get("scan_sources_sha256") != h.hexdigest():
        return None
    return int(rec["scan_traffic_bytes_per_launch"])


FP8_MFMA_PEAK_TFLOPS = 5000.0  # dense FP8 MFMA, MI355X


def inputs_digest(wl):
    """SHA-256 over one generated workload (every tensor's name, dtype,
    shape and bytes, then the other fields' reprs, in key order), so that
    runs can show they measured the same inputs. Tensors are copied to the
    host in 256 MB slices."""
    import hashlib
    import torch
    h = hashlib.sha256()
    for key in sorted(wl):
        v = wl[key]
        h.update(key.encode())
        if isinstance(v, torch.Tensor):
            h.update(f"{v.dtype}{tuple(v.shape)}".encode())
            flat = v.detach().contiguous().reshape(-1).view(torch.uint8)
            step_b = 1 << 28
            for i in range(0, flat.numel(), step_b):
                h.update(flat[i:i + step_b].cpu().numpy().tobytes())
        else:
            h.update(repr(v).encode())
    return h.hexdigest()


def prefill_indexer(dev, passes, warmup):
    """Chunked-prefill indexer: 2,048 causal query rows x 16 heads x 128 FP8
    dims against 1,048,576 index keys (the tiled MFMA kernel), then per-row
    top-2048 over the 2,048 x 1M scores, each timed over back-to-back passes
    with HIP events."""
    import torch

    import tsd_synth
    import top_sparse_decode_amd.step as step
    cfg = tsd_synth.config("qsa_prefill_r2048_l1048576_k2048")
    layer = tsd_synth.make(cfg, dev)
    bufs = step.StepBuffers(layer)
    stream = torch.cuda.current_stream()

    def timed(fn, n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n  # ms

    ms_score = timed(lambda: step.score(layer, bufs), passes)
    ms_topk = timed(lambda: step.select(layer, bufs), passes)
    ms_fused = timed(lambda: step.score_select(layer, bufs), passes)
    rows_n = (layer["q_pos"].to(torch.int64) + 1).clamp(max=cfg.L)
    flops = 2.0 * cfg.H_i * cfg.D_i * float(rows_n.sum())
    tflops = flops / (ms_score * 1e-3) / 1e12
    del bufs, layer
    torch.cuda.empty_cache()
    return {"workload": cfg.name, "rows": cfg.prefill_rows, "keys": cfg.L,
            "index_heads": cfg.H_i, "top_k": cfg.top_k,
            "flops_per_pass": flops, "score_ms": ms_score,
            "topk_ms": ms_topk, "score_topk_fused_ms": ms_fused,
            "roofline": {"bound": "mfma", "kernel": "sparse_index_score",
                         "achieved": tflops, "peak": FP8_MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s",
                         "frac": tflops / FP8_MFMA_PEAK_TFLOPS},
            "vs_target": vs_target(cfg.name, ms_score)}


def sharded_select(dev, passes, warmup, W=4):
    """Page-owner sharded exact top-k, emulated on one GPU: the 1,048,576-
    token request split over W shards (shard w owns the logical pages
    p % W == w; at W = 4 each holds 262,144 tokens, one GPU's share), each
    shard scored and selected by sparse_index_topk, then topk_merge_sharded.
    Times the whole emulated selection, the merge alone and the unsharded
    sparse_index_topk, over back-to-back passes with HIP events."""
    import torch

    import tsd_synth
    import top_sparse_decode_amd as tsd
    cfg = tsd_synth.config("qsa_decode_b1_l1048576_k2048")
    wl = tsd_synth.make(cfg, dev)
    k, B = cfg.top_k, cfg.B
    views = tsd_synth.shard_views(wl, W)
    stride = views[0]["page_table"].shape[1] * 64
    S = torch.empty((W, B, stride), device=dev)
    lens = torch.empty((W, B), dtype=torch.int32, device=dev)
    il = torch.empty((W, B, k), dtype=torch.int32, device=dev)
    cl = torch.empty((W, B), dtype=torch.int32, device=dev)
    ws = [torch.zeros(tsd.topk_select_workspace_bytes(B, stride, k),
                      dtype=torch.uint8, device=dev) for _ in range(W)]
    idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((B,), dtype=torch.int32, device=dev)
    full_stride = wl["page_table"].shape[1] * 64
    Sf = torch.empty((B, full_stride), device=dev)
    lf = torch.empty((B,), dtype=torch.int32, device=dev)
    wsf = torch.zeros(tsd.topk_select_workspace_bytes(B, full_stride, k),
                      dtype=torch.uint8, device=dev)
    idxf = torch.empty((B, k), dtype=torch.int32, device=dev)
    cntf = torch.empty((B,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def shards():
        for w, v in enumerate(views):
            tsd.sparse_index_topk("qsa", S[w], v["page_table"], v["seq_lens"],
                                  wl["num_pages"], k, il[w], cl[w], ws[w],
                                  lens[w], index_q=wl["index_q"],
                                  index_w=wl["index_w"],
                                  index_k_pool=wl["index_k"],
                                  ws_zeroed=True)

    def merge():
        tsd.topk_merge_sharded(S, il, cl, k, idx, cnt)

    def unsharded():
        tsd.sparse_index_topk("qsa", Sf, wl["page_table"], wl["seq_lens"],
                              wl["num_pages"], k, idxf, cntf, wsf, lf,
                              index_q=wl["index_q"], index_w=wl["index_w"],
                              index_k_pool=wl["index_k"], ws_zeroed=True)

    def timed(fn, n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n  # us

    us_all = timed(lambda: (shards(), merge()), passes)
    us_merge = timed(merge, passes)
    us_full = timed(unsharded, passes)
    exact = bool(torch.equal(idx, idxf) and torch.equal(cnt, cntf))
    del wl, S, Sf
    torch.cuda.empty_cache()
    return {"workload": cfg.name, "shards": W, "tokens_per_shard": stride,
            "top_k": k, "sharded_select_us": us_all, "merge_us": us_merge,
            "unsharded_select_us": us_full,
            "merge_candidates_per_row": W * k,
            "equals_unsharded": exact}


def block_select(dev, passes, warmup, Bs=4, kb=512):
    """Block-compressed QSA selection on the 262,144-token decode workload
    (8 requests): blocks of Bs tokens get one compressed FP8 index key each;
    the step scores and selects kb blocks (kb * Bs tokens) and expands them.
    Times the full compression of every cached block (once per prompt), the
    per-step compression of each request's last block, the block score+select
    and the expansion, then the attention over the expanded tokens against
    the attention on the block indices (and both chains from compression to
    attention): n back-to-back calls captured in a HIP graph, one
    replay timed with HIP events (device time, without the per-call host
    marshalling of the binding)."""
    import torch

    import tsd_synth
    import top_sparse_decode_amd as tsd
    cfg = tsd_synth.config("qsa_decode_b8_l262144_k2048")
    wl = tsd_synth.make(cfg, dev)
    B = cfg.B
    lay = tsd_synth.compressed_layout(wl, Bs)
    nblk = lay["block_lens"]
    max_blocks = int(nblk.max())
    last = (nblk - 1).clamp(min=0)
    stride = lay["cpage_table"].shape[1] * 64
    S = torch.empty((B, stride), device=dev)
    rl = torch.empty(B, dtype=torch.int32, device=dev)
    bidx = torch.empty((B, kb), dtype=torch.int32, device=dev)
    bcnt = torch.empty(B, dtype=torch.int32, device=dev)
    ws = torch.zeros(tsd.topk_select_workspace_bytes(B, stride, kb),
                     dtype=torch.uint8, device=dev)
    tok = torch.empty((B, kb * Bs), dtype=torch.int32, device=dev)
    tcnt = torch.empty(B, dtype=torch.int32, device=dev)

    def compress_all():
        tsd.index_k_compress(wl["index_k"], wl["page_table"], wl["num_pages"],
                             wl["seq_lens"], lay["ck_pool"], lay["cpage_table"],
                             lay["num_cpages"], Bs, max_blocks)

    def compress_step():
        tsd.index_k_compress(wl["index_k"], wl["page_table"], wl["num_pages"],
                             wl["seq_lens"], lay["ck_pool"], lay["cpage_table"],
                             lay["num_cpages"], Bs, 1, last)

    def select():
        tsd.sparse_index_topk("qsa", S, lay["cpage_table"], nblk,
                              lay["num_cpages"], kb, bidx, bcnt, ws, rl,
                              index_q=wl["index_q"], index_w=wl["index_w"],
                              index_k_pool=lay["ck_pool"], ws_zeroed=True)

    def expand():
        tsd.expand_blocks(bidx, bcnt, Bs, wl["seq_lens"], tok, tcnt)

    def timed(fn, n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e3 / n  # us

    us_all = timed(compress_all, max(1, passes // 10))
    us_step = timed(compress_step, passes)
    us_sel = timed(select, passes)
    us_exp = timed(expand, passes)
    us_chain = timed(lambda: (compress_step(), select(), expand()), passes)
    # the attention that consumes the selection: over the expanded tokens,
    # or directly over the block indices (idx_block), which drops the
    # expansion launch
    C = cfg.chunks
    o = torch.empty((B, cfg.H_q, C, 128), device=dev)
    lse = torch.empty((B, cfg.H_q, C), device=dev)

    def attend(ix, cn, blk):
        tsd.sparse_gqa_decode(wl["q"], wl["k_pool"], wl["v_pool"],
                              wl["page_table"], wl["seq_lens"],
                              wl["num_pages"], ix, cn, C, o, lse,
                              k_scale=wl["k_scale"], v_scale=wl["v_scale"],
                              idx_block=blk)

    tok3, tcnt2 = tok.view(B, 1, kb * Bs), tcnt.view(B, 1)
    bidx3, bcnt2 = bidx.view(B, 1, kb), bcnt.view(B, 1)
    us_att_tok = timed(lambda: attend(tok3, tcnt2, 0), passes)
    us_att_blk = timed(lambda: attend(bidx3, bcnt2, Bs), passes)
    us_step_tok = timed(lambda: (compress_step(), select(), expand(),
                                 attend(tok3, tcnt2, 0)), passes)
    us_step_blk = timed(lambda: (compress_step(), select(),
                                 attend(bidx3, bcnt2, Bs)), passes)
    tokens = float(wl["seq_lens"].to(torch.int64).sum())
    blocks = float(nblk.to(torch.int64).sum())
    comp_bytes = tokens * 128 + blocks * 128   # raw keys read, block keys written
    scan_bytes = blocks * 128                  # compressed keys read per step
    del wl, lay, S, o, lse
    torch.cuda.empty_cache()
    return {"workload": cfg.name, "block_size": Bs, "top_k_blocks": kb,
            "top_k_tokens": kb * Bs, "blocks_per_request": max_blocks,
            "compress_all_us": us_all,
            "compress_all_gbps": comp_bytes / (us_all * 1e-6) / 1e9,
            "compress_step_us": us_step, "block_select_us": us_sel,
            "block_scan_model_bytes": scan_bytes, "expand_us": us_exp,
            "block_selection_step_us": us_chain,
            "attention_expanded_us": us_att_tok,
            "attention_on_blocks_us": us_att_blk,
            "step_with_expansion_us": us_step_tok,
            "step_on_blocks_us": us_step_blk}


# Steps/s targets on one MI355X: 70 % of the HBM roofline of each decode
# workload's model bytes (index or label keys of every cached token plus the
# selected tokens' K/V), and for the prefill indexer 50 % of dense FP8 MFMA
# peak on its causal contraction (ms per pass). The tiny workload fits in the
# L2 caches and has no roofline target.
TARGETS = {"qsa_decode_b8_l262144_k2048": ("steps_per_s", 19.6e3),
           "qsa_decode_b1_l1048576_k2048": ("steps_per_s", 41.0e3),
           "ds_llama31_8b_b3_l60000": ("steps_per_s", 43.4e3),
           "ds_llama7b_b3_l20000_s200": ("steps_per_s", 50.0e3),
           "qsa_prefill_r2048_l1048576_k2048": ("score_ms", 3.5)}


def vs_target(name, value):
    """{"target": t, "unit": u, "achieved_over_target": f} (f >= 1 meets the
    target; for times, target / value), or None without a target."""
    if name not in TARGETS:
        return None
    unit, t = TARGETS[name]
    f = t / value if unit.endswith("_ms") else value / t
    return {"target": t, "unit": unit, "achieved_over_target": f}


def decode_leg(dev, name, steps, warmup, replicas=None):
    """One decode step (index or label scan + exact top-k through
    sparse_index_topk, sparse attention, LSE merge) on workload ``name``: K
    eager steps over replicas of the scanned pool (label pool for double
    sparsity, index-K for QSA; about 1 GB between two visits of a replica,
    so the Infinity Cache cannot serve the scan; K/V pools are shared, their
    gather being a small random read), then each of the four calls alone
    over back-to-back launches with HIP events. Roofline: the scanned key
    bytes of every cached token per scan launch."""
    import torch

    import tsd_synth
    import top_sparse_decode_amd.step as step
    cfg = tsd_synth.config(name)
    index_b, gather_b = model_bytes(cfg)
    R = replicas or max(1, math.ceil(1e9 / index_b))
    wl = tsd_synth.make(cfg, dev)
    pool = "label_pool" if cfg.mode == "ds" else "index_k"
    layers = [wl] + [dict(wl, **{pool: wl[pool].clone()}) for _ in range(R - 1)]
    bufs = step.StepBuffers(wl)
    plans = [step.Plan(layer, bufs, fused=True) for layer in layers]
    plans_sep = [step.Plan(layer, bufs, fused=False) for layer in layers]
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        plans[i % R].run(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        plans[i % R].run(stream)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps
    table = [dict(p.calls(stream)) for p in plans_sep]
    us = {}
    for call in ("sparse_index_score", "topk_select", "sparse_gqa_decode",
                 "lse_merge"):
        for i in range(warmup):
            plans_sep[i % R].run(stream)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            table[i % R][call]()
        e1.record(stream)
        torch.cuda.synchronize()
        us[call] = e0.elapsed_time(e1) * 1e3 / steps
    scan_us = us["sparse_index_score"]
    scan_gbps = index_b / (scan_us * 1e-6) / 1e9
    del layers, plans, plans_sep, bufs, wl
    torch.cuda.empty_cache()
    out = {"workload": name, "batch": cfg.B, "context": cfg.L,
           "H_q": cfg.H_q, "H_kv": cfg.H_kv, "top_k": cfg.top_k,
           "chunks": cfg.chunks, "kv_cache": cfg.kv_enc, "replicas": R,
           "steps_per_s": 1.0 / step_s, "ms_per_step": step_s * 1e3,
           "model_bytes_per_step": index_b + gather_b,
           "step_model_gbps": (index_b + gather_b) / step_s / 1e9,
           "scan_us": scan_us, "kernel_us": us,
           "roofline": {"bound": "hbm", "kernel": "sparse_index_score ("
                        + ("label" if cfg.mode == "ds" else "index") + " scan)",
                        "achieved": scan_gbps, "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": scan_gbps / HBM_PEAK_GBPS,
                        "bytes_per_launch": index_b}}
    if cfg.mode == "ds":
        out["heavy_channels"] = cfg.r
    out["vs_target"] = vs_target(name, out["steps_per_s"])
    return out


def tiny_leg(dev, steps, warmup):
    """The tiny double-sparsity workload (1 request, 4,096 tokens, 8 query
    heads on 1 KV head, top-256): its 262 KB per step stay in the caches,
    so it is reported as latency (us per step), one layer, eager steps."""
    out = decode_leg(dev, "ds_tiny_b1_l4096", steps, warmup, replicas=1)
    out["us_per_step"] = out["ms_per_step"] * 1e3
    out.pop("roofline", None)
    out["bound"] = "latency (working set in cache)"
    return out


def ds_append_loop(dev, warmup_loops=1, replicas=None):
    """The LLaMA-7B-shaped double-sparsity workload as the pages run it: 200
    decode steps, each first storing every request's new token (K, V and its
    label row, kv_append) and then decoding (sparse_index_topk,
    sparse_gqa_decode, lse_merge), lengths 20,001 .. 20,200, a fresh query
    per step. Each step runs on ``replicas`` layers (own label pools, shared
    K/V pools) so the label bytes read between two visits of a layer exceed
    the Infinity Cache. The timed region is the whole loop, the per-step
    query and length updates included; steps/s counts one layer's append +
    decode."""
    import torch

    import tsd_synth
    import top_sparse_decode_amd as tsd
    import top_sparse_decode_amd.step as step
    cfg = tsd_synth.config("ds_llama7b_b3_l20000_s200")
    index_b, gather_b = model_bytes(cfg)
    R = replicas or max(1, math.ceil(1e9 / index_b))
    wl = tsd_synth.make(cfg, dev)
    layers = [wl] + [dict(wl, label_pool=wl["label_pool"].clone())
                     for _ in range(R - 1)]
    bufs = step.StepBuffers(wl)
    plans = [step.Plan(layer, bufs, fused=True) for layer in layers]
    base = wl["seq_lens"].clone()
    pt = wl["page_table"]
    B, S = cfg.B, cfg.steps
    pos = (base.long() - 1)[:, None] + torch.arange(S, device=dev)[None]
    slots = pt.long().gather(1, pos // 64) * 64 + pos % 64
    k_rows = wl["k_pool"][slots].contiguous()      # [B, S, H_kv, D]
    v_rows = wl["v_pool"][slots].contiguous()
    one = torch.ones(B, dtype=torch.int32, device=dev)
    pos32 = pos.to(torch.int32)
    lens_s = [(base + s).contiguous() for s in range(S)]
    new_k = [k_rows[:, s:s + 1].contiguous() for s in range(S)]
    new_v = [v_rows[:, s:s + 1].contiguous() for s in range(S)]
    new_pos = [pos32[:, s].contiguous() for s in range(S)]
    appends = [[tsd.kv_append(pt, wl["num_pages"], new_pos[s], one, 1,
                              k_new=new_k[s], v_new=new_v[s],
                              k_pool=wl["k_pool"], v_pool=wl["v_pool"],
                              channel_idx=wl["channel_idx"],
                              label_pool=layer["label_pool"], prepare=True)
                for layer in layers] for s in range(S)]

    def loop():
        for s in range(S):
            wl["seq_lens"].copy_(lens_s[s])
            wl["q"].copy_(wl["step_q"][s])
            for li, plan in enumerate(plans):
                rc = appends[s][li]()
                if rc:
                    raise RuntimeError(f"kv_append failed: {rc}")
                plan.run()

    for _ in range(warmup_loops):
        loop()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = wall / (S * R)
    mean_len = float(base.float().mean()) + (S - 1) / 2
    label_b = B * mean_len * cfg.H_kv * cfg.r * 2
    del layers, plans, bufs, wl, k_rows, v_rows
    torch.cuda.empty_cache()
    out = {"workload": cfg.name, "batch": B, "decode_steps": S,
           "lengths": [int(base[0]), int(base[0]) + S - 1],
           "replicas": R, "steps_per_s": 1.0 / per, "us_per_step": per * 1e6,
           "tokens_per_s_per_layer": B / per,
           "model_bytes_per_step": label_b + gather_b,
           "step_model_gbps": (label_b + gather_b) / per / 1e9,
           "in_timed_region": "kv_append (K, V, label) + sparse_index_topk + "
                              "sparse_gqa_decode + lse_merge per layer, query "
                              "and length updates per step"}
    out["vs_target"] = vs_target(cfg.name, out["steps_per_s"])
    return out


def append_bench(dev, passes, warmup):
    """kv_append at decode shapes, one new token per request, timed per call
    (pre-marshalled C calls) over back-to-back launches with HIP events: the
    262,144-token FP8
    workload (8 requests, 4 KV heads: K, V with per-page scales, index-K),
    on a page the call starts and mid-page, and the 200-step double-sparsity
    workload (3 requests, 32 KV heads: FP16 K, V and the 16-channel label)."""
    import torch

    import top_sparse_decode_amd as tsd
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(passes):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / passes  # us

    out = {}
    B, H, D, P = 8, 4, 128, 4097  # 4,096 cached pages + the new tokens' page
    pt = torch.full((B, P), -1, dtype=torch.int32, device=dev)
    pt[:, P - 1] = torch.arange(B, dtype=torch.int32, device=dev)
    kp = torch.zeros((B * 64, H, D), dtype=torch.uint8, device=dev)
    vp = torch.zeros_like(kp)
    ks = torch.ones(B, device=dev)
    vs = torch.ones(B, device=dev)
    ip = torch.zeros((B * 64, 128), dtype=torch.uint8, device=dev)
    kn = torch.randn((B, 1, H, D), device=dev).to(torch.bfloat16)
    vn = torch.randn((B, 1, H, D), device=dev).to(torch.bfloat16)
    ikn = torch.randn((B, 1, 128), device=dev).to(torch.bfloat16)
    one = torch.ones(B, dtype=torch.int32, device=dev)
    for name, p0 in (("qsa_b8_fp8_new_page_us", 4096 * 64),
                     ("qsa_b8_fp8_mid_page_us", 4096 * 64 + 17)):
        pos = torch.full((B,), p0, dtype=torch.int32, device=dev)
        out[name] = timed(tsd.kv_append(
            pt, B, pos, one, 1, k_new=kn, v_new=vn, k_pool=kp, v_pool=vp,
            k_scale=ks, v_scale=vs, index_k_new=ikn, index_k_pool=ip,
            stream=stream, prepare=True))
    B, H, r, P = 3, 32, 16, 316
    pt = torch.full((B, P), -1, dtype=torch.int32, device=dev)
    pt[:, 312] = torch.arange(B, dtype=torch.int32, device=dev)
    kp = torch.zeros((B * 64, H, D), dtype=torch.float16, device=dev)
    vp = torch.zeros_like(kp)
    lp = torch.zeros((B * 64, H, r), dtype=torch.float16, device=dev)
    ch = torch.stack([torch.randperm(D, device=dev)[:r] for _ in range(H)]).to(torch.int32)
    kn = torch.randn((B, 1, H, D), device=dev).to(torch.float16)
    vn = torch.randn((B, 1, H, D), device=dev).to(torch.float16)
    pos = torch.full((B,), 20000, dtype=torch.int32, device=dev)
    one = torch.ones(B, dtype=torch.int32, device=dev)
    out["ds_b3_fp16_label_us"] = timed(tsd.kv_append(
        pt, B, pos, one, 1, k_new=kn, v_new=vn, k_pool=kp, v_pool=vp,
        channel_idx=ch, label_pool=lp, stream=stream, prepare=True))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="qsa_decode_b8_l262144_k2048")
    ap.add_argument("--replicas", type=int, default=0,
                    help="layer replicas (0: enough for >= 1 GB between reuse)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the chunked-prefill indexer measurement")
    ap.add_argument("--prefill-passes", type=int, default=5)
    ap.add_argument("--no-ds", action="store_true",
                    help="skip the double-sparsity decode measurements")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the 1,048,576-token single-request decode step")
    ap.add_argument("--no-blocks", action="store_true",
                    help="skip the block-compressed selection measurement")
    ap.add_argument("--no-tiny", action="store_true",
                    help="skip the tiny double-sparsity workload")
    ap.add_argument("--no-loop", action="store_true",
                    help="skip the 200-step append + decode loop")
    ap.add_argument("--no-sharded", action="store_true",
                    help="skip the page-owner sharded top-k emulation")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing HIP-graph replays of the step")
    ap.add_argument("--graph", action="store_true",
                    help="report HIP-graph replays of the step as the value instead of eager "
                         "launches")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the steps, copy a buffer of this many MiB "
                         "once (a plain copy kernel of known size, to scale "
                         "the HBM byte counters of a profiler run)")
    ap.add_argument("--unfused", action="store_true",
                    help="time sparse_index_score + topk_select instead of "
                         "sparse_index_topk")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU: this library has no multi-GPU path "
              "(sharding is described in the design notes); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import tsd_synth
    import top_sparse_decode_amd.step as step

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cfg = tsd_synth.config(args.workload)
    index_b, gather_b = model_bytes(cfg)
    R = args.replicas or max(1, math.ceil(1e9 / index_b))
    layers = [tsd_synth.make(cfg, dev, layer=i) for i in range(R)]
    bufs = step.StepBuffers(layers[0])
    plans = [step.Plan(layer, bufs, fused=not args.unfused) for layer in layers]
    # the instrumented pass issues the calls separately, so the events around
    # sparse_index_score bracket the scan kernel alone
    plans_sep = [step.Plan(layer, bufs, fused=False) for layer in layers]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    for i in range(args.warmup):
        plans[i % R].run(stream)
    torch.cuda.synchronize()

    K = args.steps
    # eager steps (the four C calls launched from the host each step)
    t0 = time.perf_counter()
    for i in range(K):
        plans[i % R].run(stream)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t0

    # the same step captured once per layer into a HIP graph and replayed
    graphs = []
    wall_graph = None
    if not args.no_graph or args.graph:
        for plan in plans:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                plan.run(torch.cuda.current_stream())
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            graphs[i % R].replay()
        torch.cuda.synchronize()
        wall_graph = time.perf_counter() - t0
    wall = wall_graph if args.graph else wall_eager

    # kernel durations: for each call, K back-to-back launches (rotating the
    # layers) between two HIP events on the launch stream; the average per
    # launch is the call's device time including its dispatch
    from top_sparse_decode_amd import TsdError
    names = ("sparse_index_score", "topk_select", "sparse_gqa_decode",
             "lse_merge")
    fused_plans = plans if not args.unfused else [
        step.Plan(layer, bufs, fused=True) for layer in layers]
    table = [dict(p.calls(stream)) for p in plans_sep]
    for p, f in zip(table, fused_plans):
        p["sparse_index_topk"] = dict(f.calls(stream))["sparse_index_topk"]
    us = {}
    for name in names + ("sparse_index_topk",):
        for i in range(args.warmup):
            plans_sep[i % R].run(stream)  # leave consistent buffers behind
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(K):
            rc = table[i % R][name]()
            if rc:
                raise TsdError(name, rc)
        e1.record(stream)
        torch.cuda.synchronize()
        us[name] = e0.elapsed_time(e1) * 1e3 / K

    # stream-copy bandwidth of the part (1 GiB device copy, read + write)
    del graphs
    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    big2 = torch.empty_like(big)
    big2.copy_(big)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(10):
        big2.copy_(big)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del big, big2
    torch.cuda.empty_cache()

    step_s = wall / K
    scan_s = us["sparse_index_score"] * 1e-6
    achieved = index_b / scan_s / 1e9
    line = {
        "metric": METRIC,
        "value": 1.0 / step_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if cfg.kv_enc == "fp8_e4m3" else cfg.kv_enc,
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.B, "context": cfg.L,
                   "top_k": cfg.top_k, "chunks": cfg.chunks, "H_q": cfg.H_q,
                   "H_kv": cfg.H_kv, "head_dim": cfg.D, "kv_cache": cfg.kv_enc,
                   "index_heads": cfg.H_i if cfg.mode == "qsa" else None,
                   "heavy_channels": cfg.r if cfg.mode == "ds" else None,
                   "page_size": 64, "layer_replicas": R},
        "model_bytes_per_step": index_b + gather_b,
        "step_model_gbps": (index_b + gather_b) / step_s / 1e9,
        "step_frac_of_hbm": (index_b + gather_b) / step_s / 1e9 / HBM_PEAK_GBPS,
        "kernel_us": us,
        "launch_mode": "hip_graph" if args.graph else "eager",
        "score_select": "separate calls" if args.unfused else "sparse_index_topk",
        "eager_steps_per_s": K / wall_eager,
        "graph_steps_per_s": K / wall_graph if wall_graph else None,
        "copy_gbps": copy_gbps,
        "roofline": {"bound": "hbm",
                     "kernel": ("qsa_scan_kernel<G, false> (sparse_index_score "
                                "alone; the step's sparse_index_topk runs the "
                                "same scan with the digit-1 histogram built in "
                                "LDS, <G, true>, the same bytes)"
                                if cfg.mode == "qsa" else
                                "ds_scan_vec_kernel (sparse_index_score alone)"),
                     "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "bytes_per_launch": index_b, "traffic": scan_traffic()},
    }
    line["vs_target"] = vs_target(cfg.name, line["value"])
    line["inputs_sha256"] = inputs_digest(layers[0])
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(layers[0], args.cpu_seconds)
    if not args.no_prefill:
        del plans, plans_sep, table, fused_plans, bufs, layers
        torch.cuda.empty_cache()
        line["prefill_indexer"] = prefill_indexer(dev, args.prefill_passes, 2)
    if not args.no_sharded:
        line["sharded_topk"] = sharded_select(dev, 200, 20)
    line["kv_append"] = append_bench(dev, 500, 20)
    if not args.no_long:
        line["long_decode"] = decode_leg(dev, "qsa_decode_b1_l1048576_k2048", 500, 50)
    if not args.no_ds:
        line["ds_decode"] = [decode_leg(dev, n, 500, 50) for n in
                             ("ds_llama31_8b_b3_l60000", "ds_llama7b_b3_l20000_s200")]
    if not args.no_loop:
        line["ds_append_decode_loop"] = ds_append_loop(dev)
    if not args.no_tiny:
        line["tiny_decode"] = tiny_leg(dev, 500, 50)
    if not args.no_blocks:
        line["block_compressed_select"] = block_select(dev, 200, 20)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
