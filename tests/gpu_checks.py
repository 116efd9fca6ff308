"""Comparisons of the HIP path against the CPU oracle, shared by the GPU
tests, the smoke check and the benchmark's spot checks.

Tolerances (max absolute error, FP32 accumulation on both sides):
  scores:  2e-3 for double-sparsity labels in BF16/FP16, 2e-2 for FP8 index
           keys;
  outputs and LSEs: 2e-3 for a BF16/FP16 cache, 2e-2 for an FP8 cache;
  top-k:   identical index arrays when both sides see the same f32 scores;
           end to end, the selected sets may differ only among tokens whose
           oracle score lies within 1e-5 * max(1, |s_k|) of the k-th score
           s_k, and the set sizes must agree.
Where the two selections differ, attention is compared with the oracle run
on the GPU's own selection, so the numerics of the gather and the softmax
are always checked element by element.
"""
from __future__ import annotations

import numpy as np

import oracle

TIE_WINDOW = 1e-5


def score_tol(mode):
    return 2e-3 if mode == "ds" else 2e-2


def out_tol(kv_enc):
    return 2e-2 if kv_enc == "fp8_e4m3" else 2e-3


def oracle_scores(h):
    if h["mode"] == "ds":
        return oracle.ds_scores(h["q"], h["q_enc"], h["channel_idx"],
                                h["label_pool"], h["kv_enc"], h["page_table"],
                                h["seq_lens"], h["num_pages"])
    return oracle.qsa_scores(h["index_q"], h["index_w"], h["index_k"],
                             h["page_table"], h["seq_lens"], h["num_pages"],
                             rows_per_req=h.get("rows_per_req", 1),
                             q_pos=h.get("q_pos"))


def oracle_row_lens(h):
    lens = h["seq_lens"].astype(np.int64)
    if h["mode"] == "ds":
        return np.repeat(lens, h["channel_idx"].shape[0])
    R = h.get("rows_per_req", 1)
    rl = np.repeat(lens, R)
    if h.get("q_pos") is not None:
        rl = np.minimum(rl, np.maximum(h["q_pos"].astype(np.int64) + 1, 0))
    return rl


def check_scores(gpu, ref64, row_lens, tol, rows=None):
    """Entries t < n agree within tol; the rest of each row is untouched
    (the GPU buffer was pre-filled with NaN)."""
    rows = range(gpu.shape[0]) if rows is None else rows
    worst = 0.0
    for r in rows:
        n = int(row_lens[r])
        g = gpu[r, :n].astype(np.float64)
        assert np.isfinite(g).all(), f"row {r}: non-finite score"
        err = np.abs(g - ref64[r, :n]).max() if n else 0.0
        worst = max(worst, err)
        assert err <= tol, f"row {r}: score error {err}"
        assert np.isnan(gpu[r, n:]).all(), f"row {r}: tail written"
    return worst


def score_error_vs_window(gpu, ref64, row_lens, k):
    """Per row: the largest score error over the row divided by the tie
    window 1e-5 * max(1, |s_k|) of its k-th oracle score. When twice that
    error fits in the window, every end-to-end selection difference is a
    near-tie by construction (a swap of t and u needs both within two error
    bounds of s_k), whatever the data. Returns the per-row ratios."""
    out = []
    for r in range(gpu.shape[0]):
        n = int(row_lens[r])
        if n == 0:
            out.append(0.0)
            continue
        ref = ref64[r, :n]
        m = min(k, n)
        sk = np.partition(ref.astype(np.float32).astype(np.float64), n - m)[n - m]
        err = np.abs(gpu[r, :n].astype(np.float64) - ref).max()
        out.append(err / (TIE_WINDOW * max(1.0, abs(sk))))
    return np.array(out)


def check_topk_identical(scores32, row_lens, k, gpu_idx, gpu_count, rows=None):
    """Same f32 scores in -> identical arrays out."""
    rows = np.arange(scores32.shape[0]) if rows is None else np.asarray(rows)
    ref_idx, ref_cnt = oracle.topk(scores32[rows], row_lens[rows], k)
    np.testing.assert_array_equal(gpu_count[rows], ref_cnt)
    np.testing.assert_array_equal(gpu_idx[rows], ref_idx)


def check_sets_within_window(gpu_idx, gpu_cnt, ref_idx, ref_cnt, ref_s32,
                             row_lens, k, rows=None, label=""):
    """End-to-end selections: equal sizes, differences only at near-ties.
    Every array is aligned row by row; ``rows`` only names the rows in the
    printout (default 0, 1, ...).
    Prints, per row, the size of the symmetric difference, the largest
    distance of a differing token's oracle score from the k-th score s_k
    (in units of the window 1e-5 * max(1, |s_k|)) and the oracle's own gap
    between the k-th and the (k+1)-th score. Returns the number of rows
    whose sets differ."""
    rows = range(gpu_idx.shape[0]) if rows is None else rows
    differing = 0
    for i, r in enumerate(rows):
        n = int(row_lens[i])
        assert gpu_cnt[i] == ref_cnt[i] == min(k, n)
        m = int(ref_cnt[i])
        a = set(gpu_idx[i, :m].tolist())
        b = set(ref_idx[i, :m].tolist())
        assert (gpu_idx[i, m:] == -1).all()
        assert (np.diff(gpu_idx[i, :m]) > 0).all()
        s = ref_s32[i, :n].astype(np.float64)
        srt = np.sort(s)[::-1]
        sk = srt[m - 1] if m else 0.0
        gap = (srt[m - 1] - srt[m]) if m < n else float("inf")
        window = TIE_WINDOW * max(1.0, abs(sk))
        diff = a ^ b
        far = max((abs(s[t] - sk) for t in diff), default=0.0)
        print(f"sets {label} row {r}: n={n} k={m} differing={len(diff)} "
              f"max|s_t-s_k|/window={far / window:.3g} s_k={sk:.6g} "
              f"gap(k,k+1)={gap:.3g}", flush=True)
        if diff:
            differing += 1
            for t in diff:
                assert abs(s[t] - sk) <= window, (r, t, s[t], sk)
    return differing


def check_attention_on(h, idx3, cnt2, chunks, o_part, lse_part, tol,
                       batch=None):
    """Oracle attention on the GPU's selection vs the GPU partials."""
    bsel = np.arange(h["q"].shape[0]) if batch is None else np.asarray(batch)
    sub = dict(h)
    sub["q"] = h["q"][bsel]
    sub["page_table"] = h["page_table"][bsel]
    sub["seq_lens"] = h["seq_lens"][bsel]
    ro, rl = oracle.sparse_attention(
        sub["q"], h["q_enc"], h["k_pool"], h["v_pool"], h["kv_enc"],
        h.get("k_scale"), h.get("v_scale"), sub["page_table"], sub["seq_lens"],
        h["num_pages"], idx3[bsel], cnt2[bsel], chunks)
    go = o_part[bsel].astype(np.float64)
    gl = lse_part[bsel].astype(np.float64)
    assert (np.isneginf(gl) == np.isneginf(rl)).all(), "empty chunks differ"
    fin = np.isfinite(rl)
    err_o = np.abs(go - ro).max()
    err_l = np.abs(gl[fin] - rl[fin]).max() if fin.any() else 0.0
    assert err_o <= tol, f"o_part error {err_o}"
    assert err_l <= tol, f"lse_part error {err_l}"
    return ro, rl, max(err_o, err_l)


def check_merge(o_part, lse_part, out, out_lse, tol=1e-5):
    """GPU merge vs oracle merge of the GPU's own partials."""
    C, D = o_part.shape[-2], o_part.shape[-1]
    ro, rl = oracle.lse_merge(o_part.reshape(-1, C, D).astype(np.float64),
                              lse_part.reshape(-1, C).astype(np.float64))
    go = out.reshape(-1, D).astype(np.float64)
    gl = out_lse.reshape(-1).astype(np.float64)
    assert (np.isneginf(gl) == np.isneginf(rl)).all()
    fin = np.isfinite(rl)
    err = max(np.abs(go - ro).max(),
              np.abs(gl[fin] - rl[fin]).max() if fin.any() else 0.0)
    assert err <= tol, f"merge error {err}"
    return err


# ------------------------------------------------ page-owner sharded select
def gpu_topk_stack(S, lens, kl):
    """topk_select on each shard's [rows, stride] scores (one call per
    shard) -> idx [W, rows, kl], count [W, rows] on the scores' device."""
    import torch
    import top_sparse_decode_amd as tsd
    W, rows, stride = S.shape
    idx = torch.full((W, rows, kl), -7, dtype=torch.int32, device=S.device)
    cnt = torch.full((W, rows), -7, dtype=torch.int32, device=S.device)
    ws = torch.empty(tsd.topk_select_workspace_bytes(rows, stride, kl),
                     dtype=torch.uint8, device=S.device)
    for w in range(W):
        tsd.topk_select(S[w], lens[w], kl, stride, idx[w], cnt[w], ws)
    return idx, cnt


def sharded_qsa_select(wl, W, k):
    """Every page-owner shard scores and selects over its own pages of a QSA
    decode workload; the candidates are merged. Returns (idx [B, k], count
    [B], shard scores [W, B, stride_w], shard lengths [W, B])."""
    import torch
    import top_sparse_decode_amd as tsd
    import tsd_synth
    views = tsd_synth.shard_views(wl, W)
    B = wl["page_table"].shape[0]
    dev = wl["page_table"].device
    stride = views[0]["page_table"].shape[1] * 64
    S = torch.full((W, B, stride), float("nan"), device=dev)
    lens = torch.empty((W, B), dtype=torch.int32, device=dev)
    for w, v in enumerate(views):
        tsd.sparse_index_score("qsa", S[w], v["page_table"], v["seq_lens"],
                               wl["num_pages"], index_q=wl["index_q"],
                               index_w=wl["index_w"],
                               index_k_pool=wl["index_k"], row_lens_out=lens[w])
    il, cl = gpu_topk_stack(S, lens, k)
    idx = torch.empty((B, k), dtype=torch.int32, device=dev)
    cnt = torch.empty((B,), dtype=torch.int32, device=dev)
    tsd.topk_merge_sharded(S, il, cl, k, idx, cnt)
    return idx, cnt, S, lens
