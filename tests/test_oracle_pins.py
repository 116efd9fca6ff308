"""Pins of the CPU oracle against things other than itself: format
definitions and library conversions, hand-worked fixtures, brute force on tiny
inputs, closed forms and invariants. Each test is chosen so that a plausible
mistake in the oracle (a dropped term, a wrong sign or index, a transposed
operand, a wrong tie rule) fails it. CPU only."""
import math
import os

import numpy as np
import pytest
import torch

import tsd_synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- decoders
def test_fp8_golden_points(orc):
    for line in open(os.path.join(GOLDEN, "fp8_e4m3_ocp.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = orc.decode_fp8_e4m3(int(code, 16))
        if val == "nan":
            assert math.isnan(got), code
        else:
            assert got == float(val), code
            assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


def test_fp8_exhaustive_against_torch(orc):
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.decode_fp8_e4m3(c) for c in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert nan.sum() == 2  # 0x7F and 0xFF only
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.nanmax(np.abs(got)) == 448.0


def test_bf16_exhaustive_against_torch(orc):
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([orc.decode_bf16(c) for c in range(65536)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert np.array_equal(got[~nan], ref[~nan])


def test_fp16_exhaustive_against_numpy(orc):
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    ref = ref.astype(np.float64)
    got = np.array([orc.decode_fp16(c) for c in range(65536)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------------------- slot mapping
def _golden_slots():
    rows = []
    for line in open(os.path.join(GOLDEN, "slot_mapping.txt")):
        if line.startswith("#") or not line.strip():
            continue
        rows.append(tuple(int(x) for x in line.split()))
    return rows


PT_GOLDEN = np.array([[3, 0, 2], [1, 4, 5]], np.int32)


def test_slot_golden(orc):
    for b, t, want in _golden_slots():
        assert orc.slot(PT_GOLDEN, b, t, 64, 6) == want
    assert orc.slot(np.array([[9]], np.int32), 0, 5, 64, 6) == -1
    assert orc.slot(np.array([[-1]], np.int32), 0, 5, 64, 6) == -1


def test_ds_scores_read_the_mapped_slot(orc):
    """Label value = its own slot number (exact in fp16); one channel, unit
    query -> each score must be the golden slot of that token."""
    slots = 6 * 64
    label = torch.arange(slots, dtype=torch.float32).to(torch.float16)
    label = label.view(slots, 1, 1).view(torch.int16).numpy().view(np.uint16)
    q = torch.zeros(2, 1, 4, dtype=torch.float16)
    q[:, 0, 2] = 1.0
    qc = q.view(torch.int16).numpy().view(np.uint16)
    chan = np.array([[2]], np.int32)
    lens = np.array([192, 192], np.int32)
    s = orc.ds_scores(qc, "fp16", chan, label, "fp16", PT_GOLDEN, lens, 6)
    for b, t, want in _golden_slots():
        assert s[b, t] == want


def test_ds_scores_stop_at_length_and_skip_stale_tail(orc):
    label = np.ones((6 * 64, 1, 1), np.uint16) * 0x3C00  # fp16 1.0
    q = np.ones((1, 1, 1), np.uint16) * 0x3C00
    pt = np.array([[3, 99, -4]], np.int32)  # only page 3 is live
    s = orc.ds_scores(q, "fp16", np.array([[0]], np.int32), label, "fp16",
                      pt, np.array([10], np.int32), 6, score_stride=20)
    assert (s[0, :10] == 1.0).all() and np.isnan(s[0, 10:]).all()


# ------------------------------------------------------------------- scores
def _f64(t):
    return t.to(torch.float64).numpy()


def _ident_cfg(**kw):
    base = dict(name="pin", mode="qsa", B=2, L=200, H_q=8, H_kv=2, D=32,
                top_k=16, chunks=3, kv_enc="fp8_e4m3", seed=11, H_i=4, D_i=32)
    base.update(kw)
    return tsd_synth.Config(**base)


def _identity_pages(wl):
    """Rewrite a workload so request b's pages are physically contiguous and
    in order (slot of token t of request b = b * cap * 64 + t)."""
    pt = wl["page_table"].clone()
    B, cap = pt.shape
    perm_slots = []
    for b in range(B):
        for j in range(cap):
            p = int(pt[b, j])
            perm_slots.extend(range(p * 64, p * 64 + 64))
            pt[b, j] = b * cap + j
    idx = torch.tensor(perm_slots)
    out = dict(wl)
    for key in ("index_k", "k_pool", "v_pool", "label_pool"):
        if key in wl and wl[key] is not None:
            out[key] = wl[key][idx].contiguous()
    pages = idx.view(-1, 64)[:, 0] // 64
    for key in ("k_scale", "v_scale"):
        if wl.get(key) is not None:
            out[key] = wl[key][pages].contiguous()
    out["page_table"] = pt
    return out


def test_qsa_scores_brute_force_einsum(orc):
    wl = tsd_synth.make(_ident_cfg(lens=(200, 77)))
    h = tsd_synth.to_host(wl)
    s = orc.qsa_scores(h["index_q"], h["index_w"], h["index_k"],
                       h["page_table"], h["seq_lens"], h["num_pages"])
    iq = _f64(wl["index_q"].view(torch.float8_e4m3fn))
    ik = _f64(wl["index_k"].view(torch.float8_e4m3fn))
    w = wl["index_w"].to(torch.float64).numpy()
    for b in range(2):
        n = int(wl["seq_lens"][b])
        t = np.arange(n)
        slots = wl["page_table"][b].numpy()[t // 64] * 64 + t % 64
        dots = np.einsum("hd,td->ht", iq[b], ik[slots])
        ref = np.einsum("h,ht->t", w[b], np.maximum(dots, 0.0))
        np.testing.assert_allclose(s[b, :n], ref, rtol=1e-13, atol=1e-12)


def test_qsa_special_cases(orc):
    # one head, unit weight, positive dots: the score is the plain dot product
    D = 16
    one = 0x38  # fp8 1.0
    iq = np.full((1, 1, D), one, np.uint8)
    ik = np.zeros((64, D), np.uint8)
    vals = torch.tensor([0.5, 1.0, 2.0, 3.0]).to(torch.float8_e4m3fn).view(torch.uint8)
    for t in range(64):
        ik[t] = vals[t % 4].item()
    w = np.ones((1, 1), np.float32)
    pt = np.zeros((1, 1), np.int32)
    s = orc.qsa_scores(iq, w, ik, pt, np.array([64], np.int32), 1)
    assert np.array_equal(s[0], [D * [0.5, 1, 2, 3][t % 4] for t in range(64)])
    # negative dots are cut to zero by the ReLU, whatever the weight
    ikn = ik | 0x80
    s = orc.qsa_scores(iq, w * 5, ikn, pt, np.array([64], np.int32), 1)
    assert (s[0] == 0.0).all()
    # two heads: only the positive head contributes, scaled by its weight
    iq2 = np.stack([np.full(D, one, np.uint8), np.full(D, one | 0x80, np.uint8)])[None]
    w2 = np.array([[0.25, 7.0]], np.float32)
    s = orc.qsa_scores(iq2, w2, ik, pt, np.array([64], np.int32), 1)
    assert np.array_equal(s[0], [0.25 * D * [0.5, 1, 2, 3][t % 4] for t in range(64)])


def test_qsa_causal_rows(orc):
    wl = tsd_synth.make(_ident_cfg(B=1, lens=(150,), rows_per_req=1))
    h = tsd_synth.to_host(wl)
    R = 3
    iq = np.repeat(h["index_q"], R, axis=0)
    iw = np.repeat(h["index_w"], R, axis=0)
    qpos = np.array([0, 63, 149], np.int32)
    s = orc.qsa_scores(iq, iw, h["index_k"], h["page_table"], h["seq_lens"],
                       h["num_pages"], rows_per_req=R, q_pos=qpos)
    full = orc.qsa_scores(h["index_q"], h["index_w"], h["index_k"],
                          h["page_table"], h["seq_lens"], h["num_pages"])
    for i, p in enumerate(qpos):
        assert np.array_equal(s[i, :p + 1], full[0, :p + 1])
        assert np.isnan(s[i, p + 1:]).all()


def test_score_points_match_full(orc):
    wl = tsd_synth.make(_ident_cfg(lens=(200, 77)))
    h = tsd_synth.to_host(wl)
    full = orc.qsa_scores(h["index_q"], h["index_w"], h["index_k"],
                          h["page_table"], h["seq_lens"], h["num_pages"])
    rows = np.array([0, 1, 0, 1]); ts = np.array([0, 76, 199, 3])
    pts = orc.qsa_score_points(h["index_q"], h["index_w"], h["index_k"],
                               h["page_table"], h["seq_lens"], h["num_pages"],
                               rows, ts)
    assert np.array_equal(pts, full[rows, ts])
    with pytest.raises(orc.OracleError):
        orc.qsa_score_points(h["index_q"], h["index_w"], h["index_k"],
                             h["page_table"], h["seq_lens"], h["num_pages"],
                             np.array([1]), np.array([77]))


def _ds_cfg(**kw):
    base = dict(name="pin", mode="ds", B=2, L=300, H_q=8, H_kv=2, D=32,
                top_k=20, chunks=3, kv_enc="bf16", seed=5, r=6, n_outlier=3,
                outlier_scale=6.0)
    base.update(kw)
    return tsd_synth.Config(**base)


def test_ds_scores_brute_force(orc):
    wl = tsd_synth.make(_ds_cfg(lens=(300, 65)))
    h = tsd_synth.to_host(wl)
    s = orc.ds_scores(h["q"], "bf16", h["channel_idx"], h["label_pool"],
                      "bf16", h["page_table"], h["seq_lens"], h["num_pages"])
    q = _f64(wl["q"]); lab = _f64(wl["label_pool"])
    ch = wl["channel_idx"].numpy()
    G = 4
    for b in range(2):
        n = int(wl["seq_lens"][b])
        t = np.arange(n)
        slots = wl["page_table"][b].numpy()[t // 64] * 64 + t % 64
        for g in range(2):
            qs = q[b, g * G:(g + 1) * G][:, ch[g]].sum(axis=0)
            ref = lab[slots, g, :] @ qs
            np.testing.assert_allclose(s[b * 2 + g, :n], ref, rtol=1e-13,
                                       atol=1e-12)


def test_ds_score_points_brute_force(orc):
    """Point-wise label scores (the oracle's checker for sampled entries of
    long rows): row = b * H_kv + g. Random (row, t) pairs over 3 requests of
    2 KV heads each are compared with a numpy brute force of the label score
    at that point (the group's summed query at the heavy channels dotted
    with the label of the token's mapped slot) and with the full score
    matrix; a pair past its row's length or a row outside [0, B * H_kv)
    raises."""
    wl = tsd_synth.make(_ds_cfg(B=3, lens=(300, 65, 130)))
    h = tsd_synth.to_host(wl)
    q = _f64(wl["q"]); lab = _f64(wl["label_pool"])
    ch = wl["channel_idx"].numpy()
    pt = wl["page_table"].numpy()
    lens = wl["seq_lens"].numpy()
    H_kv, G = 2, 4
    rng = np.random.default_rng(3)
    rows = rng.integers(0, 3 * H_kv, size=200)
    ts = np.array([rng.integers(0, lens[r // H_kv]) for r in rows])
    rows[:6], ts[:6] = np.arange(6), lens[np.arange(6) // H_kv] - 1
    pts = orc.ds_score_points(h["q"], "bf16", h["channel_idx"], h["label_pool"],
                              "bf16", h["page_table"], h["seq_lens"],
                              h["num_pages"], rows, ts)
    for i, (r, t) in enumerate(zip(rows, ts)):
        b, g = divmod(int(r), H_kv)
        slot = pt[b, t // 64] * 64 + t % 64
        qs = q[b, g * G:(g + 1) * G][:, ch[g]].sum(axis=0)
        assert abs(pts[i] - lab[slot, g, :] @ qs) <= 1e-12 * max(1, abs(pts[i]))
    full = orc.ds_scores(h["q"], "bf16", h["channel_idx"], h["label_pool"],
                         "bf16", h["page_table"], h["seq_lens"], h["num_pages"])
    assert np.array_equal(pts, full[rows, ts])
    for bad_r, bad_t in ((1, 300), (2, 65), (6, 0), (-1, 0)):
        with pytest.raises(orc.OracleError):
            orc.ds_score_points(h["q"], "bf16", h["channel_idx"],
                                h["label_pool"], "bf16", h["page_table"],
                                h["seq_lens"], h["num_pages"],
                                np.array([bad_r]), np.array([bad_t]))


def test_ds_full_channels_give_group_logits(orc):
    """r = D with identity channels: the label score is (sum of the group's
    query heads) . K_t, i.e. the group's summed attention logits."""
    wl = tsd_synth.make(_ds_cfg(r=32, lens=(130, 64)))
    h = tsd_synth.to_host(wl)
    assert (h["channel_idx"] == np.arange(32)).all()
    s = orc.ds_scores(h["q"], "bf16", h["channel_idx"], h["label_pool"],
                      "bf16", h["page_table"], h["seq_lens"], h["num_pages"])
    q = _f64(wl["q"]); k = _f64(wl["k_pool"])
    for b in range(2):
        for g in range(2):
            n = int(wl["seq_lens"][b])
            t = np.arange(n)
            slots = wl["page_table"][b].numpy()[t // 64] * 64 + t % 64
            logits = np.einsum("hd,td->ht", q[b, g * 4:(g + 1) * 4], k[slots, g])
            np.testing.assert_allclose(s[b * 2 + g, :n], logits.sum(0),
                                       rtol=1e-12, atol=1e-10)


def test_scores_invariant_under_page_permutation(orc):
    wl = tsd_synth.make(_ident_cfg(lens=(200, 77)))
    wi = _identity_pages(wl)
    a, b = tsd_synth.to_host(wl), tsd_synth.to_host(wi)
    sa = orc.qsa_scores(a["index_q"], a["index_w"], a["index_k"],
                        a["page_table"], a["seq_lens"], a["num_pages"])
    sb = orc.qsa_scores(b["index_q"], b["index_w"], b["index_k"],
                        b["page_table"], b["seq_lens"], b["num_pages"])
    assert np.array_equal(np.nan_to_num(sa, nan=-1), np.nan_to_num(sb, nan=-1))


# -------------------------------------------------------------------- top-k
def _brute_topk(s, k):
    order = sorted(range(len(s)), key=lambda t: (-s[t], t))[:k]
    out = sorted(order)
    return out + [-1] * (k - len(out))


def test_topk_brute_force_small(orc):
    rng = np.random.default_rng(0)
    values = np.array([-np.inf, -2.0, -0.0, 0.0, 0.5, 1.0, 1.0, np.inf],
                      np.float32)
    for trial in range(300):
        n = int(rng.integers(0, 11))
        s = rng.choice(values, size=max(n, 1)).astype(np.float32)[:n]
        for k in range(1, 12):
            idx, cnt = orc.topk(np.pad(s, (0, 12 - n))[None], [n], k)
            assert list(idx[0]) == _brute_topk(list(s), k)
            assert cnt[0] == min(k, n)


def test_topk_invariants_random(orc):
    rng = np.random.default_rng(1)
    for n, k in [(5000, 100), (4096, 256), (300, 300), (100, 1000)]:
        s = rng.normal(size=n).astype(np.float32)
        s[rng.integers(0, n, 50)] = s[7]  # ties, some at the threshold
        idx, cnt = orc.topk(s[None], [n], k)
        m = min(k, n)
        sel = idx[0, :m]
        assert cnt[0] == m and (idx[0, m:] == -1).all()
        assert (np.diff(sel) > 0).all()
        mask = np.zeros(n, bool); mask[sel] = True
        if m < n:
            thr = s[mask].min()
            assert thr >= s[~mask].max()
            ties_in = np.where(mask & (s == thr))[0]
            ties_out = np.where(~mask & (s == thr))[0]
            if len(ties_out):
                assert ties_in.max() < ties_out.min()


def test_topk_signed_zero_tie_and_empty_rows(orc):
    s = np.array([[-0.0, 0.0, -0.0, 0.0]], np.float32)
    idx, cnt = orc.topk(s, [4], 2)
    assert list(idx[0]) == [0, 1]  # -0 and +0 are one value: lowest indices win
    idx, cnt = orc.topk(np.zeros((2, 4), np.float32), [0, -3], 3)
    assert (idx == -1).all() and (cnt == 0).all()
    with pytest.raises(orc.OracleError):
        orc.topk(np.array([[1.0, np.nan]], np.float32), [2], 1)


def _sharded_topk(orc, s, n, W, k, page_size=64, kl=None):
    """Shard a row by page owner p % W, select k locally per shard with the
    oracle top-k, and merge the candidates with the oracle merge."""
    kl = k if kl is None else kl
    orders = orc.shard_row_order(n, W, page_size)
    L = max(1, max(len(o) for o in orders))
    S = np.zeros((W, 1, L), np.float32)
    I = np.zeros((W, 1, kl), np.int32)
    C = np.zeros((W, 1), np.int32)
    for w, o in enumerate(orders):
        S[w, 0, :len(o)] = s[o]
        I[w], C[w] = orc.topk(S[w], [len(o)], kl)
    return orc.topk_merge_sharded(S, I, C, k, page_size)


def test_sharded_merge_hand_worked(orc):
    # page size 2, W = 2: shard 0 owns pages 0 and 2 (tokens 0,1,4,5), shard 1
    # owns page 1 (tokens 2,3); local token u of shard 1 is global u + 2
    s = np.array([5.0, 1.0, 5.0, 7.0, 1.0, 5.0], np.float32)
    idx, cnt = _sharded_topk(orc, s, 6, 2, 3, page_size=2)
    assert list(idx[0]) == [0, 2, 3] and cnt[0] == 3  # 7, then 5s at 0 and 2
    idx, cnt = _sharded_topk(orc, s, 6, 2, 4, page_size=2)
    assert list(idx[0]) == [0, 2, 3, 5]
    # a shard's local token maps back through its page: u = 2 of shard 0 is
    # token 4 (page 2), u = 1 of shard 1 is token 3
    S = np.array([[[0, 0, 9, 0]], [[0, 8, 0, 0]]], np.float32)
    I = np.array([[[2]], [[1]]], np.int32)
    C = np.array([[1], [1]], np.int32)
    idx, cnt = orc.topk_merge_sharded(S, I, C, 2, page_size=2)
    assert list(idx[0]) == [3, 4] and cnt[0] == 2


@pytest.mark.parametrize("W", [1, 2, 3, 4, 5])
def test_sharded_merge_equals_unsharded(orc, W):
    # the global top-k of a row lies in the union of the shards' local
    # top-ks, with the lowest global token winning ties across shards
    rng = np.random.default_rng(W)
    for n, k, levels in [(1000, 50, 20), (5000, 300, 3), (64 * 7 + 5, 100, 4),
                         (40, 100, 5), (130, 7, 1), (20000, 2048, 1000)]:
        s = (rng.integers(0, levels, size=n) / levels).astype(np.float32)
        s[rng.random(n) < 0.05] = -0.0
        got, gc = _sharded_topk(orc, s, n, W, k)
        ref, rc = orc.topk(s[None], [n], k)
        np.testing.assert_array_equal(got, ref)
        np.testing.assert_array_equal(gc, rc)


def test_sharded_merge_short_local_lists(orc):
    # local lists shorter than k (kl < k) still merge exactly when every
    # shard keeps at least its share of the global top-k
    rng = np.random.default_rng(11)
    n, W, k = 4096, 4, 64
    s = rng.normal(size=n).astype(np.float32)
    got, _ = _sharded_topk(orc, s, n, W, k, kl=k)
    ref, _ = orc.topk(s[None], [n], k)
    np.testing.assert_array_equal(got, ref)
    # an empty row and rows shorter than one page per shard
    got, gc = _sharded_topk(orc, s, 0, W, k)
    assert (got == -1).all() and gc[0] == 0
    got, gc = _sharded_topk(orc, s, 70, W, k)
    ref, rc = orc.topk(s[None, :70], [70], k)
    np.testing.assert_array_equal(got, ref)


# -------------------------------------------------------------- cache append
def test_fp8_encode_round_trips_every_code(orc):
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue  # the NaN codes
        assert orc.encode_fp8_e4m3(orc.decode_fp8_e4m3(c)) == c, c


def test_fp8_encode_midpoints_saturation_and_torch(orc):
    pos = [orc.decode_fp8_e4m3(c) for c in range(0x7F)]
    for c in range(0x7E):
        mid = (pos[c] + pos[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert orc.encode_fp8_e4m3(mid) == even
        assert orc.encode_fp8_e4m3(-mid) == 0x80 | even
        assert orc.encode_fp8_e4m3(np.nextafter(mid, 1e9)) == c + 1
    for x, code in [(448.0, 0x7E), (463.9, 0x7E), (1e9, 0x7E), (-600.0, 0xFE),
                    (0.0, 0x00), (-0.0, 0x80), (-1e-30, 0x80), (2.0 ** -10, 0x00),
                    (3 * 2.0 ** -10, 0x02)]:
        assert orc.encode_fp8_e4m3(x) == code, x
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.normal(size=4000) * 40, rng.normal(size=2000) * 1e-2,
                        rng.uniform(-447, 447, 2000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.encode_fp8_e4m3(float(v)) for v in x], np.uint8)
    np.testing.assert_array_equal(got, ref)


def _bf16_codes(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def test_append_16bit_rows_label_and_index(orc):
    # 2 requests, page table with a bad page id and a short capacity
    rng = np.random.default_rng(4)
    H, D, r, slots = 2, 8, 3, 6 * 64
    pt = np.array([[3, 1, -1], [0, 5, 2]], np.int32)
    kp = rng.integers(0, 65535, (slots, H, D)).astype(np.uint16)
    vp = rng.integers(0, 65535, (slots, H, D)).astype(np.uint16)
    lp = rng.integers(0, 65535, (slots, H, r)).astype(np.uint16)
    ip = rng.integers(0, 255, (slots, 16)).astype(np.uint8)
    kn = _bf16_codes(rng.normal(size=(2, 5, H, D)))
    vn = _bf16_codes(rng.normal(size=(2, 5, H, D)))
    ikn = rng.normal(size=(2, 5, 16)).astype(np.float32) * 30
    ch = np.array([[0, 5, 7], [2, 3, 6]], np.int32)
    positions, n_new = [62, 190], [5, 3]
    got = orc.kv_append(pt, 6, positions, n_new, 5, k_new=kn, v_new=vn,
                        k_pool=kp, v_pool=vp, channel_idx=ch, label_pool=lp,
                        index_k_new=ikn, index_enc="f32", index_k_pool=ip)
    # request 0: positions 62, 63 on page 3; 64, 65, 66 on page 1
    # request 1: 190, 191 on page 2 (logical page 2); 192 is past capacity
    writes = {(0, 0): 3 * 64 + 62, (0, 1): 3 * 64 + 63, (0, 2): 64 + 0,
              (0, 3): 64 + 1, (0, 4): 64 + 2, (1, 0): 2 * 64 + 62,
              (1, 1): 2 * 64 + 63}
    ek, ev, el, ei = kp.copy(), vp.copy(), lp.copy(), ip.copy()
    for (b, i), slot in writes.items():
        ek[slot], ev[slot] = kn[b, i], vn[b, i]
        el[slot] = np.take_along_axis(kn[b, i], ch, axis=1)
        ei[slot] = torch.from_numpy(ikn[b, i]).to(torch.float8_e4m3fn).view(
            torch.uint8).numpy()
    np.testing.assert_array_equal(got["k_pool"], ek)
    np.testing.assert_array_equal(got["v_pool"], ev)
    np.testing.assert_array_equal(got["label_pool"], el)
    np.testing.assert_array_equal(got["index_k_pool"], ei)
    assert got["k_scale"] is None


def test_append_fp8_pages_match_the_page_quantizer(orc):
    # a call that fills a fresh page gives the per-page quantization of the
    # workload generator (scale = amax/448 in f32, round to nearest even); a
    # page it starts but does not fill gets four times that range
    rng = np.random.default_rng(5)
    H, D = 2, 16
    x = (rng.normal(size=(1, 64 + 10, H, D)) * 3).astype(np.float32)
    x[0, 64:] *= 5
    xb = torch.from_numpy(x).to(torch.bfloat16)
    kn = xb.view(torch.int16).numpy().view(np.uint16)
    pt = np.array([[2, 0]], np.int32)
    kp = np.zeros((3 * 64, H, D), np.uint8)
    ks = np.full(3, 7.0, np.float32)
    got = orc.kv_append(pt, 3, [0], [74], 74, k_new=kn, v_new=kn,
                        k_pool=kp, v_pool=kp.copy(), kv_enc="fp8_e4m3",
                        k_scale=ks, v_scale=ks.copy())
    # the full page: the generator's page quantizer (amax / 448)
    pad = xb[0, 0:64].float()
    codes, scale = tsd_synth.quantize_fp8_per_page(pad)
    assert got["k_scale"][2] == scale[0].item()
    np.testing.assert_array_equal(got["k_pool"][2 * 64:3 * 64], codes.numpy())
    # the page the call leaves unfinished (10 of 64 tokens): 4 x amax / 448,
    # codes = torch's float8 cast of value / scale, saturating at 448
    vals = xb[0, 64:74].float()
    s4 = np.float32(np.float32(vals.abs().max().item()) / np.float32(448.0)) * np.float32(4.0)
    assert got["k_scale"][0] == s4
    q = torch.clamp(vals / torch.tensor(s4), -448.0, 448.0).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(got["k_pool"][0:10], q.view(torch.uint8).numpy())
    assert got["k_scale"][1] == 7.0  # untouched page keeps its scale
    # appending to a started page keeps its scale and saturates above 448*s
    kn2 = _bf16_codes(np.full((1, 1, H, D), 1e4))
    got2 = orc.kv_append(pt, 3, [74], [1], 1, k_new=kn2, v_new=kn2,
                         k_pool=got["k_pool"], v_pool=got["v_pool"],
                         kv_enc="fp8_e4m3", k_scale=got["k_scale"],
                         v_scale=got["v_scale"])
    # token 74 is on logical page 1 = physical page 0, slot 10
    assert got2["k_scale"][0] == got["k_scale"][0]
    assert (got2["k_pool"][10] == 0x7E).all()
    keep = np.ones(3 * 64, bool)
    keep[10] = False
    np.testing.assert_array_equal(got2["k_pool"][keep], got["k_pool"][keep])


# ------------------------------------------------------ block compression
def _fp8_decode_np(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def _compress_case(orc, lens, Bs, seed, from_block=None):
    rng = np.random.default_rng(seed)
    B = len(lens)
    P = max(1, -(-max(lens) // 64))
    num_pages = B * P + 2
    pt = rng.permutation(num_pages)[:B * P].reshape(B, P).astype(np.int32)
    ik = rng.integers(0, 0x7E, size=(num_pages * 64, 128)).astype(np.uint8)
    ik |= (rng.random(ik.shape) < 0.5).astype(np.uint8) << 7
    nblk = [-(-n // Bs) for n in lens]
    CP = max(1, -(-max(nblk) // 64))
    num_cpages = B * CP + 1
    cpt = rng.permutation(num_cpages)[:B * CP].reshape(B, CP).astype(np.int32)
    ck0 = rng.integers(0, 255, size=(num_cpages * 64, 128)).astype(np.uint8)
    fb = np.zeros(B, np.int32) if from_block is None else np.asarray(from_block, np.int32)
    ck = orc.index_k_compress(ik, pt, num_pages, lens, fb, cpt, num_cpages,
                              ck0, Bs)
    return pt, ik, cpt, ck0, ck, fb, nblk


def test_compress_block_size_one_is_the_token_keys(orc):
    lens = [200, 64, 1]
    pt, ik, cpt, _, ck, _, _ = _compress_case(orc, lens, 1, 20)
    for b, n in enumerate(lens):
        for t in range(n):
            slot = pt[b, t // 64] * 64 + t % 64
            cslot = cpt[b, t // 64] * 64 + t % 64
            if ik[slot].tolist() != ck[cslot].tolist():
                # -0 and +0 are one value: the mean of -0 is +0
                assert (_fp8_decode_np(ik[slot]) == _fp8_decode_np(ck[cslot])).all()


def test_compress_means_match_numpy(orc):
    lens, Bs = [1000, 70, 5], 16
    pt, ik, cpt, ck0, ck, fb, nblk = _compress_case(orc, lens, Bs, 21,
                                                    from_block=[3, 0, 0])
    for b, n in enumerate(lens):
        for j in range(nblk[b]):
            cslot = cpt[b, j // 64] * 64 + j % 64
            if j < fb[b]:
                np.testing.assert_array_equal(ck[cslot], ck0[cslot])
                continue
            ts = np.arange(j * Bs, min((j + 1) * Bs, n))
            slots = pt[b, ts // 64] * 64 + ts % 64
            mean = _fp8_decode_np(ik[slots]).mean(axis=0).astype(np.float32)
            ref = torch.from_numpy(mean).to(torch.float8_e4m3fn).view(
                torch.uint8).numpy()
            got_v = _fp8_decode_np(ck[cslot])
            ref_v = _fp8_decode_np(ref)
            np.testing.assert_array_equal(got_v, ref_v)


def test_compress_hand_worked_ties_and_bad_pages(orc):
    one, two, three, four = (orc.encode_fp8_e4m3(x) for x in (1, 2, 3, 4))
    ik = np.zeros((2 * 64, 128), np.uint8)
    ik[0:4, 0] = [one, two, three, four]      # mean 2.5 (exact)
    ik[0:4, 1] = [one, one, one, two]         # mean 1.25 (exact)
    ik[4:8, 2] = [one, one, one, orc.encode_fp8_e4m3(1.25)]  # 1.0625: tie -> 1
    pt = np.array([[0, 7]], np.int32)         # page 7 is outside the pool
    cpt = np.array([[1]], np.int32)
    ck0 = np.full((2 * 64, 128), 0x11, np.uint8)
    ck = orc.index_k_compress(ik, pt, 2, [70], [0], cpt, 2, ck0, 4)
    assert ck[64, 0] == orc.encode_fp8_e4m3(2.5)
    assert ck[64, 1] == orc.encode_fp8_e4m3(1.25)
    assert ck[65, 2] == one
    # block 16 (tokens 64..67) sits on page 7: not written
    assert (ck[64 + 16] == 0x11).all()


def test_expand_blocks_hand_worked(orc):
    sel = np.array([[0, 2, 5, -1], [1, 0, 0, 0]], np.int32)
    tok, cnt = orc.expand_blocks(sel, [3, 1], 4, [22, 3], 12)
    assert tok[0].tolist() == [0, 1, 2, 3, 8, 9, 10, 11, 20, 21, -1, -1]
    assert cnt[0] == 10
    assert tok[1].tolist() == [-1] * 12 and cnt[1] == 0  # block 1 is past len 3
    tok, cnt = orc.expand_blocks(sel, [3, 1], 4, [22, 8], 6)
    assert tok[0].tolist() == [0, 1, 2, 3, 8, 9] and cnt[0] == 6
    assert tok[1].tolist() == [4, 5, 6, 7, -1, -1] and cnt[1] == 4


def test_block_pipeline_with_block_size_one_is_the_token_pipeline(orc):
    # Bs = 1: compress, score the blocks, select, expand == score, select
    cfg = _ident_cfg(mode="qsa", B=2, L=300, lens=(300, 130), D_i=128, H_i=4,
                     top_k=40, seed=30)
    wl = tsd_synth.to_host(tsd_synth.make(cfg))
    s_tok = orc.qsa_scores(wl["index_q"], wl["index_w"], wl["index_k"],
                           wl["page_table"], wl["seq_lens"], wl["num_pages"])
    i_tok, c_tok = orc.topk(s_tok.astype(np.float32), wl["seq_lens"], 40)
    ck = orc.index_k_compress(wl["index_k"], wl["page_table"], wl["num_pages"],
                              wl["seq_lens"], [0, 0], wl["page_table"],
                              wl["num_pages"], np.zeros_like(wl["index_k"]), 1)
    s_blk = orc.qsa_scores(wl["index_q"], wl["index_w"], ck, wl["page_table"],
                           wl["seq_lens"], wl["num_pages"])
    i_blk, c_blk = orc.topk(s_blk.astype(np.float32), wl["seq_lens"], 40)
    tok, cnt = orc.expand_blocks(i_blk, c_blk, 1, wl["seq_lens"], 40)
    np.testing.assert_array_equal(tok, i_tok)
    np.testing.assert_array_equal(cnt, c_tok)


# ---------------------------------------------------------------- attention
def _decoded_kv(wl, key, scale_key):
    x = wl[key]
    if x.dtype == torch.uint8:
        v = x.view(torch.float8_e4m3fn).to(torch.float64)
        sc = wl[scale_key].to(torch.float64)
        v = v * sc.repeat_interleave(64)[:, None, None]
        return v
    return x.to(torch.float64)


def _attn_case(kv_enc, lens, **kw):
    cfg = _ident_cfg(kv_enc=kv_enc, lens=lens, D=64, **kw)
    wl = tsd_synth.make(cfg)
    if kv_enc != "fp8_e4m3":
        wl["q_enc"] = kv_enc
    return wl


def _all_selected(wl):
    B = wl["B"]
    n = int(wl["seq_lens"].max())
    idx = np.full((B, 1, n), -1, np.int32)
    cnt = np.zeros((B, 1), np.int32)
    for b in range(B):
        lb = int(wl["seq_lens"][b])
        idx[b, 0, :lb] = np.arange(lb)
        cnt[b, 0] = lb
    return idx, cnt


@pytest.mark.parametrize("kv_enc", ["fp8_e4m3", "bf16"])
def test_full_selection_is_dense_attention_sdpa(orc, kv_enc):
    wl = _attn_case(kv_enc, (200, 77))
    h = tsd_synth.to_host(wl)
    idx, cnt = _all_selected(wl)
    o, lse = orc.sparse_attention(h["q"], h["q_enc"], h["k_pool"], h["v_pool"],
                                  h["kv_enc"], h.get("k_scale"),
                                  h.get("v_scale"), h["page_table"],
                                  h["seq_lens"], h["num_pages"], idx, cnt, 1)
    dense, dlse = orc.dense_attention(h["q"], h["q_enc"], h["k_pool"],
                                      h["v_pool"], h["kv_enc"],
                                      h.get("k_scale"), h.get("v_scale"),
                                      h["page_table"], h["seq_lens"],
                                      h["num_pages"])
    np.testing.assert_allclose(o[:, :, 0], dense, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[:, :, 0], dlse, rtol=0, atol=1e-12)
    # independent reference: torch SDPA on CPU float64 over decoded values
    K = _decoded_kv(wl, "k_pool", "k_scale")
    V = _decoded_kv(wl, "v_pool", "v_scale")
    q = wl["q"].to(torch.float64)
    G = wl["H_q"] // wl["H_kv"]
    for b in range(wl["B"]):
        n = int(wl["seq_lens"][b])
        t = torch.arange(n)
        slots = wl["page_table"][b].long()[t // 64] * 64 + t % 64
        Kb = K[slots].permute(1, 0, 2).repeat_interleave(G, 0)  # [H_q, n, D]
        Vb = V[slots].permute(1, 0, 2).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[b][:, None, :], Kb, Vb)[:, 0]
        np.testing.assert_allclose(o[b, :, 0], ref.numpy(), rtol=0, atol=1e-12)
        logits = (q[b][:, None, :] @ Kb.transpose(1, 2))[:, 0] / math.sqrt(wl["D"])
        np.testing.assert_allclose(lse[b, :, 0],
                                   torch.logsumexp(logits, -1).numpy(),
                                   rtol=0, atol=1e-12)


def test_single_token_and_identical_keys(orc):
    wl = _attn_case("bf16", (130,), B=1)
    h = tsd_synth.to_host(wl)
    V = _decoded_kv(wl, "v_pool", None).numpy()
    K = _decoded_kv(wl, "k_pool", None).numpy()
    q = wl["q"].to(torch.float64).numpy()
    pt = h["page_table"]
    t = 70
    slot = pt[0, t // 64] * 64 + t % 64
    idx = np.array([[[t]]], np.int32)
    o, lse = orc.sparse_attention(h["q"], "bf16", h["k_pool"], h["v_pool"],
                                  "bf16", None, None, pt, h["seq_lens"],
                                  h["num_pages"], idx, np.array([[1]]), 1)
    G = 4
    for hq in range(wl["H_q"]):
        assert np.array_equal(o[0, hq, 0], V[slot, hq // G])
        z = q[0, hq] @ K[slot, hq // G] / math.sqrt(wl["D"])
        assert abs(lse[0, hq, 0] - z) < 1e-12
    # identical keys: uniform weights, output = mean of the values
    kp = h["k_pool"].copy()
    sel = [3, 64, 100, 129]
    slots = [pt[0, s // 64] * 64 + s % 64 for s in sel]
    for s in slots:
        kp[s] = kp[slots[0]]
    o, lse = orc.sparse_attention(h["q"], "bf16", kp, h["v_pool"], "bf16",
                                  None, None, pt, h["seq_lens"],
                                  h["num_pages"], np.array([[sel]], np.int32),
                                  np.array([[4]]), 1)
    for hq in range(wl["H_q"]):
        np.testing.assert_allclose(o[0, hq, 0], V[slots, hq // G].mean(0),
                                   rtol=0, atol=1e-12)


def test_constant_values_give_constant_output(orc):
    wl = _attn_case("fp8_e4m3", (190, 64))
    h = tsd_synth.to_host(wl)
    vp = np.full_like(h["v_pool"], 0x38)  # every value 1.0 before scaling
    vs = np.full_like(h["v_scale"], 0.75)
    idx, cnt = _all_selected(wl)
    o, lse = orc.sparse_attention(h["q"], "bf16", h["k_pool"], vp, "fp8_e4m3",
                                  h["k_scale"], vs, h["page_table"],
                                  h["seq_lens"], h["num_pages"], idx, cnt, 4)
    np.testing.assert_allclose(o, 0.75, rtol=0, atol=1e-12)


# -------------------------------------------------------------------- merge
@pytest.mark.parametrize("C", [1, 2, 3, 7, 16, 64, 190])
def test_any_chunk_split_merges_to_unsplit(orc, C):
    wl = _attn_case("fp8_e4m3", (190, 64))
    h = tsd_synth.to_host(wl)
    idx, cnt = _all_selected(wl)
    args = (h["q"], "bf16", h["k_pool"], h["v_pool"], "fp8_e4m3", h["k_scale"],
            h["v_scale"], h["page_table"], h["seq_lens"], h["num_pages"], idx,
            cnt)
    o1, l1 = orc.sparse_attention(*args, 1)
    oc, lc = orc.sparse_attention(*args, C)
    B, H = o1.shape[:2]
    out, lse = orc.lse_merge(oc.reshape(B * H, C, -1), lc.reshape(B * H, C))
    np.testing.assert_allclose(out, o1[:, :, 0].reshape(B * H, -1), rtol=0,
                               atol=1e-12)
    np.testing.assert_allclose(lse, l1[:, :, 0].ravel(), rtol=0, atol=1e-12)
    if C > 64:  # request 1 has 64 tokens: some chunks are empty
        assert np.isinf(lc[1]).any() and (oc[1][np.isinf(lc[1])] == 0).all()


def test_random_uneven_cuts_merge_to_unsplit(orc):
    wl = _attn_case("bf16", (190,), B=1)
    h = tsd_synth.to_host(wl)
    rng = np.random.default_rng(3)
    full = np.arange(190, dtype=np.int32)
    base = (h["q"], "bf16", h["k_pool"], h["v_pool"], "bf16", None, None,
            h["page_table"], h["seq_lens"], h["num_pages"])
    o1, l1 = orc.sparse_attention(*base, full[None, None], np.array([[190]]), 1)
    for _ in range(5):
        cuts = np.sort(rng.choice(np.arange(1, 190), size=6, replace=False))
        segs = np.split(full, cuts)
        parts = [orc.sparse_attention(*base, s[None, None].copy(),
                                      np.array([[len(s)]]), 1) for s in segs]
        op = np.stack([p[0][0, :, 0] for p in parts], axis=1)  # [H, C, D]
        lp = np.stack([p[1][0, :, 0] for p in parts], axis=1)
        out, lse = orc.lse_merge(op, lp)
        np.testing.assert_allclose(out, o1[0, :, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, l1[0, :, 0], rtol=0, atol=1e-12)


def test_merge_empty_and_identity(orc):
    o = np.random.default_rng(0).normal(size=(3, 1, 8))
    l = np.array([[0.3], [-2.0], [5.0]])
    out, lse = orc.lse_merge(o, l)
    assert np.array_equal(out, o[:, 0]) and np.array_equal(lse, l[:, 0])
    out, lse = orc.lse_merge(np.ones((1, 4, 8)), np.full((1, 4), -np.inf))
    assert (out == 0).all() and lse[0] == -np.inf
    # an empty chunk next to a real one leaves the real one unchanged
    o2 = np.concatenate([o[:1], np.zeros((1, 1, 8))], axis=1)
    out, lse = orc.lse_merge(o2, np.array([[0.3, -np.inf]]))
    assert np.array_equal(out[0], o[0, 0]) and lse[0] == 0.3


def test_empty_request_gives_empty_chunks(orc):
    wl = _attn_case("fp8_e4m3", (0, 64))
    h = tsd_synth.to_host(wl)
    idx, cnt = _all_selected(wl)
    o, lse = orc.sparse_attention(h["q"], "bf16", h["k_pool"], h["v_pool"],
                                  "fp8_e4m3", h["k_scale"], h["v_scale"],
                                  h["page_table"], h["seq_lens"],
                                  h["num_pages"], idx, cnt, 2)
    assert (o[0] == 0).all() and np.isneginf(lse[0]).all()
    assert np.isfinite(lse[1]).all()


# ---------------------------------------------------------- whole decode step
def test_decode_step_topk_at_least_context_is_dense(orc):
    cfg = _ident_cfg(lens=(150, 90), top_k=256, chunks=5, D=64)
    wl = tsd_synth.make(cfg)
    h = tsd_synth.to_host(wl)
    r = orc.decode_step(h)
    dense, dlse = orc.dense_attention(h["q"], "bf16", h["k_pool"], h["v_pool"],
                                      "fp8_e4m3", h["k_scale"], h["v_scale"],
                                      h["page_table"], h["seq_lens"],
                                      h["num_pages"])
    np.testing.assert_allclose(r["out"], dense, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["out_lse"], dlse, rtol=0, atol=1e-12)
    assert list(r["count"].ravel()) == [150, 90]


def test_chunk_partition_hand_worked(orc):
    """10 selected tokens in 4 chunks are cut into contiguous runs of 2, 3, 2
    and 3 entries of the ascending list (hand-worked from the balanced
    partition floor(c*m/C)); each partial is attention over its run alone."""
    wl = _attn_case("bf16", (190,), B=1)
    h = tsd_synth.to_host(wl)
    sel = np.array([1, 5, 9, 40, 63, 64, 100, 120, 150, 189], np.int32)
    runs = [sel[0:2], sel[2:5], sel[5:7], sel[7:10]]
    base = (h["q"], "bf16", h["k_pool"], h["v_pool"], "bf16", None, None,
            h["page_table"], h["seq_lens"], h["num_pages"])
    o4, l4 = orc.sparse_attention(*base, sel[None, None], np.array([[10]]), 4)
    for c, run in enumerate(runs):
        o1, l1 = orc.sparse_attention(*base, run[None, None].copy(),
                                      np.array([[len(run)]]), 1)
        assert np.array_equal(o4[0, :, c], o1[0, :, 0])
        assert np.array_equal(l4[0, :, c], l1[0, :, 0])
