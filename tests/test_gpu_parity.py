"""GPU parity of every step of the path against the CPU oracle, through the
C ABI (via the thin binding), at sizes the oracle finishes in seconds: several
pages and tiles, ragged tails, empty requests, stale page-table tails,
partial index-head sets, causal prefill rows, ties and special values."""
import numpy as np
import pytest
import torch

import oracle
import tsd_synth
from gpu_checks import (check_attention_on, check_merge, check_scores,
                        check_sets_within_window, check_topk_identical,
                        gpu_topk_stack, oracle_row_lens, oracle_scores,
                        out_tol, score_tol, sharded_qsa_select)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import top_sparse_decode_amd  # noqa: F401  fails loudly without the library


def _step():
    import top_sparse_decode_amd.step as step
    return step


def _run(wl):
    step = _step()
    bufs = step.StepBuffers(wl)
    bufs.scores.fill_(float("nan"))
    step.decode_step(wl, bufs)
    torch.cuda.synchronize()
    return bufs


def _full_check(cfg, **over):
    print(f"case {cfg.name} B={cfg.B} lens={cfg.lens} k={cfg.top_k} "
          f"C={cfg.chunks} {cfg.kv_enc}", flush=True)
    wl = tsd_synth.make(cfg, DEV)
    wl.update(over)
    bufs = _run(wl)
    h = tsd_synth.to_host(wl)
    B, k, C = wl["B"], wl["top_k"], wl["chunks"]
    rl = oracle_row_lens(h)
    np.testing.assert_array_equal(bufs.row_lens.cpu().numpy(), rl)
    gs = bufs.scores.cpu().numpy()
    ref64 = oracle_scores(h)
    check_scores(gs, ref64, rl, score_tol(wl["mode"]))
    gidx, gcnt = bufs.idx.cpu().numpy(), bufs.count.cpu().numpy()
    check_topk_identical(gs, rl, k, gidx, gcnt)
    ref32 = ref64.astype(np.float32)
    ridx, rcnt = oracle.topk(np.nan_to_num(ref32, nan=0.0), rl, k)
    check_sets_within_window(gidx, gcnt, ridx, rcnt, ref32, rl, k)
    H_sel = bufs.H_sel
    op, lp = bufs.o_part.cpu().numpy(), bufs.lse_part.cpu().numpy()
    check_attention_on(h, gidx.reshape(B, H_sel, k), gcnt.reshape(B, H_sel), C,
                       op, lp, out_tol(wl["kv_enc"]))
    check_merge(op, lp, bufs.out.cpu().numpy(), bufs.out_lse.cpu().numpy())
    if (gidx == ridx).all():
        ref = oracle.decode_step(h)
        err = np.abs(bufs.out.cpu().numpy() - ref["out"]).max()
        assert err <= out_tol(wl["kv_enc"]), err
    return wl, bufs


QSA = "qsa_decode_b8_l262144_k2048"
DS8B = "ds_llama31_8b_b3_l60000"
DS7B = "ds_llama7b_b3_l20000_s200"


@pytest.mark.parametrize("lens,k,C", [
    ((5000, 4097, 63), 256, 5),
    ((1000, 0, 130), 300, 3),
    ((64, 65, 128), 64, 1),
    ((2048, 700), 2048, 16),
    # 32 rows of a 4,096-page table: 4,096 scan waves of 32 pages
    ((262144,) + tuple((i * 997) % 9000 for i in range(1, 32)), 256, 4),
    # the largest k and chunk count the contract takes, on a chunked-top-k row
    ((40000, 9000), 4096, 64),
])
def test_qsa_decode_path(lens, k, C):
    cfg = tsd_synth.config(QSA, B=len(lens), lens=lens, top_k=k, chunks=C,
                           seed=101)
    _full_check(cfg)


def test_qsa_stale_page_table_tail():
    cfg = tsd_synth.config(QSA, B=2, lens=(700, 129), top_k=100, chunks=4,
                           stale_tail=True, seed=102)
    _full_check(cfg)


@pytest.mark.parametrize("first", [5000, 40000], ids=["short", "long"])
def test_qsa_invalid_pages_inside_rows_score_minus_inf(first):
    """Page-table entries inside a row's length that are negative or past
    the pool: those tokens score -inf (the scan never reads them), every
    other score matches the oracle on the original table, and the fused
    selection equals the top-k of those scores (short rows: the
    one-workgroup top-k; long rows: the in-scan digit-1 histogram, which
    counts the -inf scores, then the filter and the resolve)."""
    import top_sparse_decode_amd as tsd
    cfg = tsd_synth.config(QSA, B=2, lens=(first, 300), top_k=256, chunks=4,
                           seed=104)
    wl = tsd_synth.make(cfg, DEV)
    h = tsd_synth.to_host(wl)
    ref = oracle_scores(h)
    pt = wl["page_table"].clone()
    bad = [(0, 3, -1), (0, 10, wl["num_pages"] + 7), (0, 31, -9), (0, 32, -1),
           (1, 2, wl["num_pages"])]
    for r, c, v in bad:
        pt[r, c] = v
    B, k = cfg.B, cfg.top_k
    stride = pt.shape[1] * 64
    S = torch.full((B, stride), float("nan"), device=DEV)
    rl = torch.empty(B, dtype=torch.int32, device=DEV)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    cnt = torch.empty(B, dtype=torch.int32, device=DEV)
    ws = torch.empty(tsd.topk_select_workspace_bytes(B, stride, k),
                     dtype=torch.uint8, device=DEV)
    tsd.sparse_index_topk("qsa", S, pt, wl["seq_lens"], wl["num_pages"], k,
                          idx, cnt, ws, rl, index_q=wl["index_q"],
                          index_w=wl["index_w"], index_k_pool=wl["index_k"])
    torch.cuda.synchronize()
    gs = S.cpu().numpy()
    lens = h["seq_lens"]
    mask = np.zeros_like(gs, dtype=bool)
    for r, c, _ in bad:
        mask[r, c * 64:(c + 1) * 64] = True
    for r in range(B):
        n = int(lens[r])
        bad_r = mask[r, :n]
        assert np.isneginf(gs[r, :n][bad_r]).all()
        err = np.abs(gs[r, :n][~bad_r] - ref[r, :n][~bad_r]).max()
        assert err <= score_tol("qsa"), err
        assert np.isnan(gs[r, n:]).all()
    check_topk_identical(gs, lens.astype(np.int64), k, idx.cpu().numpy(),
                         cnt.cpu().numpy())


@pytest.mark.parametrize("first", [3000, 40000], ids=["short", "long"])
def test_qsa_empty_pool_scores_minus_inf(first):
    """num_pages = 0: every token is on a page outside the pool, so every
    score is -inf and the selection is the first k tokens (lowest index
    among equal scores); the pool is never read. Long rows take the in-scan
    digit-1 histogram (every score in one bin), the filter and the resolve,
    whose ties at T are kept by index."""
    import top_sparse_decode_amd as tsd
    cfg = tsd_synth.config(QSA, B=3, lens=(first, 100, 0), top_k=128, chunks=2,
                           seed=105)
    wl = tsd_synth.make(cfg, DEV)
    B, k = cfg.B, cfg.top_k
    stride = wl["page_table"].shape[1] * 64
    S = torch.full((B, stride), float("nan"), device=DEV)
    rl = torch.empty(B, dtype=torch.int32, device=DEV)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    cnt = torch.empty(B, dtype=torch.int32, device=DEV)
    ws = torch.empty(tsd.topk_select_workspace_bytes(B, stride, k),
                     dtype=torch.uint8, device=DEV)
    tsd.sparse_index_topk("qsa", S, wl["page_table"], wl["seq_lens"], 0, k,
                          idx, cnt, ws, rl, index_q=wl["index_q"],
                          index_w=wl["index_w"], index_k_pool=wl["index_k"])
    torch.cuda.synchronize()
    gs, gi, gc = S.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()
    for r, n in enumerate(cfg.lens):
        assert np.isneginf(gs[r, :n]).all() and np.isnan(gs[r, n:]).all()
        m = min(n, k)
        assert gc[r] == m
        np.testing.assert_array_equal(gi[r, :m], np.arange(m))
        assert (gi[r, m:] == -1).all()


def test_qsa_partial_index_heads():
    cfg = tsd_synth.config(QSA, B=2, lens=(900, 333), top_k=128, chunks=2,
                           H_i=5, seed=103)
    _full_check(cfg)


def test_qsa_causal_prefill_rows():
    cfg = tsd_synth.config(QSA, B=1, lens=(1500,), top_k=200, chunks=4,
                           seed=104)
    wl = tsd_synth.make(cfg, DEV)
    R = 6
    qpos = torch.tensor([0, 63, 64, 199, 1000, 1499], dtype=torch.int32,
                        device=DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    iq = tsd_synth.fp8_codes(torch.randn((R, 16, 128), generator=g, device=DEV))
    iw = torch.rand((R, 16), generator=g, device=DEV)
    wl.update(index_q=iq, index_w=iw, rows_per_req=R, q_pos=qpos)
    step = _step()
    bufs = step.StepBuffers(wl)
    bufs.scores.fill_(float("nan"))
    step.score(wl, bufs)
    step.select(wl, bufs)
    torch.cuda.synchronize()
    h = tsd_synth.to_host(wl)
    rl = oracle_row_lens(h)
    np.testing.assert_array_equal(bufs.row_lens.cpu().numpy(), rl)
    gs = bufs.scores.cpu().numpy()
    check_scores(gs, oracle_scores(h), rl, score_tol("qsa"))
    check_topk_identical(gs, rl, 200, bufs.idx.cpu().numpy(),
                         bufs.count.cpu().numpy())


@pytest.mark.parametrize("name,over", [
    (DS8B, dict(B=2, lens=(3000, 700), top_k=200, chunks=3)),
    (DS7B, dict(B=3, H_q=6, H_kv=6, lens=(1500, 64, 65), top_k=100, chunks=4,
                steps=0)),
    (DS8B, dict(B=2, lens=(777, 300), r=12, n_outlier=12, top_k=64, chunks=2)),
    ("ds_tiny_b1_l4096", dict(lens=(4096,))),
    (DS8B, dict(B=2, lens=(2000, 900), top_k=128, chunks=3, channel_type="q")),
    (DS8B, dict(B=2, lens=(2000, 900), top_k=128, chunks=3, channel_type="qk")),
    (DS8B, dict(B=2, lens=(5000, 333), r=64, n_outlier=40, top_k=150, chunks=3)),
    (DS8B, dict(B=1, H_q=8, H_kv=4, lens=(4100,), r=128, n_outlier=16, top_k=90,
                chunks=2)),
    (DS7B, dict(B=2, H_q=12, H_kv=12, lens=(9000, 130), top_k=300, chunks=5,
                steps=0)),
    # the largest k and chunk count, rows past the one-workgroup top-k
    (DS8B, dict(B=2, lens=(40000, 5000), top_k=4096, chunks=64)),
])
def test_ds_decode_path(name, over):
    cfg = tsd_synth.config(name, seed=111, **over)
    _full_check(cfg)


@pytest.mark.parametrize("H_q,H_kv,r,lens", [
    (32, 32, 32, (3000, 77)),    # H_kv*r = 1,024: 4 sub-blocks of a page, one per workgroup
    (48, 24, 32, (2000, 129)),   # 768: 3 sub-blocks, runs of pages, two register buffers
    (32, 8, 32, (200000,)),      # 3,125 pages: two pages per workgroup
])
def test_ds_label_scan_vector_layouts(H_q, H_kv, r, lens):
    """The label scan's vector layouts beyond the workloads' (one sub-block
    per workgroup at four sub-blocks per page, page runs with three, runs of
    two pages on a long row), every score against the oracle."""
    import top_sparse_decode_amd as tsd
    cfg = tsd_synth.config(DS8B, B=len(lens), H_q=H_q, H_kv=H_kv, r=r,
                           n_outlier=r, lens=lens, top_k=64, chunks=2,
                           seed=117 + H_kv)
    wl = tsd_synth.make(cfg, DEV)
    h = tsd_synth.to_host(wl)
    ref = oracle_scores(h)
    stride = wl["page_table"].shape[1] * 64
    S = torch.full((cfg.B * H_kv, stride), float("nan"), device=DEV)
    rl = torch.empty(cfg.B * H_kv, dtype=torch.int32, device=DEV)
    tsd.sparse_index_score("ds", S, wl["page_table"], wl["seq_lens"], wl["num_pages"],
                           q=wl["q"], channel_idx=wl["channel_idx"],
                           label_pool=wl["label_pool"], row_lens_out=rl)
    torch.cuda.synchronize()
    want = np.repeat(np.array(lens), H_kv)
    np.testing.assert_array_equal(rl.cpu().numpy(), want)
    check_scores(S.cpu().numpy(), ref, want, score_tol("ds"))


@pytest.mark.parametrize("enc", ["fp16", "bf16"])
@pytest.mark.parametrize("r", [8, 16, 32, 64, 128])
@pytest.mark.parametrize("H_kv", [8, 24])
def test_ds_label_scan_types_and_label_widths(enc, r, H_kv):
    """Both 16-bit label types at every vector width of a label (r / 8
    lanes per label, 1 .. 16, their partial dots added across lanes), with
    a head count that keeps every lane on one head (8) and one that does
    not (24), two query heads per KV head: every score against the
    oracle."""
    import top_sparse_decode_amd as tsd
    lens = (1500, 77)
    cfg = tsd_synth.config(DS8B, B=len(lens), H_q=2 * H_kv, H_kv=H_kv, r=r,
                           n_outlier=r, lens=lens, kv_enc=enc, top_k=64,
                           chunks=2, seed=131 + r + H_kv)
    wl = tsd_synth.make(cfg, DEV)
    h = tsd_synth.to_host(wl)
    ref = oracle_scores(h)
    stride = wl["page_table"].shape[1] * 64
    S = torch.full((cfg.B * H_kv, stride), float("nan"), device=DEV)
    rl = torch.empty(cfg.B * H_kv, dtype=torch.int32, device=DEV)
    tsd.sparse_index_score("ds", S, wl["page_table"], wl["seq_lens"], wl["num_pages"],
                           q=wl["q"], channel_idx=wl["channel_idx"],
                           label_pool=wl["label_pool"], row_lens_out=rl)
    torch.cuda.synchronize()
    want = np.repeat(np.array(lens), H_kv)
    np.testing.assert_array_equal(rl.cpu().numpy(), want)
    check_scores(S.cpu().numpy(), ref, want, score_tol("ds"))


def test_ds_stale_tail_and_empty_request():
    cfg = tsd_synth.config(DS8B, B=3, lens=(0, 1000, 65), top_k=128, chunks=3,
                           stale_tail=True, seed=112)
    _full_check(cfg)


def test_ds_invalid_pages_inside_rows_score_minus_inf():
    """Label scan with page ids inside a row's length that are negative or
    past the pool: every head's score is -inf on those pages, every other
    score matches the oracle on the original page table."""
    import top_sparse_decode_amd as tsd
    cfg = tsd_synth.config(DS8B, B=2, lens=(9000, 500), top_k=64, chunks=2,
                           seed=113)
    wl = tsd_synth.make(cfg, DEV)
    h = tsd_synth.to_host(wl)
    ref = oracle_scores(h)
    pt = wl["page_table"].clone()
    bad = [(0, 0, -1), (0, 77, wl["num_pages"] + 3), (0, 140, -2),
           (1, 7, wl["num_pages"])]
    for r, c, v in bad:
        pt[r, c] = v
    H = cfg.H_kv
    stride = pt.shape[1] * 64
    S = torch.full((cfg.B * H, stride), float("nan"), device=DEV)
    rl = torch.empty(cfg.B * H, dtype=torch.int32, device=DEV)
    tsd.sparse_index_score("ds", S, pt, wl["seq_lens"], wl["num_pages"],
                           q=wl["q"], channel_idx=wl["channel_idx"],
                           label_pool=wl["label_pool"], row_lens_out=rl)
    torch.cuda.synchronize()
    gs = S.cpu().numpy()
    for b in range(cfg.B):
        n = int(h["seq_lens"][b])
        m = np.zeros(n, dtype=bool)
        for r, c, _ in bad:
            if r == b:
                m[c * 64:min(n, (c + 1) * 64)] = True
        for g in range(H):
            row = b * H + g
            assert np.isneginf(gs[row, :n][m]).all()
            err = np.abs(gs[row, :n][~m] - ref[row, :n][~m]).max()
            assert err <= score_tol("ds"), err
            assert np.isnan(gs[row, n:]).all()


# --------------------------------------------------------------- top-k only
def _topk_gpu(scores_np, lens, k, max_len=None):
    import top_sparse_decode_amd as tsd
    rows, stride = scores_np.shape
    max_len = stride if max_len is None else max_len
    s = torch.from_numpy(scores_np).to(DEV)
    rl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    idx = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(tsd.topk_select_workspace_bytes(rows, max_len, k),
                     dtype=torch.uint8, device=DEV)
    tsd.topk_select(s, rl, k, max_len, idx, cnt, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


def _hist_words(ws, rows):
    return ws.view(torch.int32)[:rows * 5120].cpu().numpy()


def test_topk_reuses_a_zeroed_workspace():
    """Every call leaves the histogram words zero (a garbage workspace
    without the flag, then a chain of flagged calls on the same workspace
    over inputs that take the blind, staged and raw-reread paths, short and
    empty rows, and fewer rows), each result equal to the oracle's."""
    import top_sparse_decode_amd as tsd
    rng = np.random.default_rng(77)
    rows0, stride, k = 6, 70000, 2048
    ws = torch.full((tsd.topk_select_workspace_bytes(rows0, stride, k),), 0xAB,
                    dtype=torch.uint8, device=DEV)
    cases = []
    s = rng.normal(size=(rows0, stride)).astype(np.float32)
    cases.append((s, [stride, 60000, 2048, 2047, 0, 30000], False))
    t = (rng.integers(0, 40, size=(rows0, stride)) / 40).astype(np.float32)
    cases.append((t, [stride] * rows0, True))          # heavy ties
    u = rng.normal(size=(rows0, stride)).astype(np.float32)
    u[1, 4096:8192] += 20.0                             # one overflowing chunk
    u[2, ::3] = 5.0                                     # many ties at the top
    cases.append((u, [stride, stride, 50000, 100, 1, 69999], True))
    v = rng.normal(size=(3, stride)).astype(np.float32)
    cases.append((v, [65000, 2049, 40000], True))      # fewer rows
    for sc, lens, zeroed in cases:
        r = sc.shape[0]
        idx = torch.full((r, k), -7, dtype=torch.int32, device=DEV)
        cnt = torch.full((r,), -7, dtype=torch.int32, device=DEV)
        tsd.topk_select(torch.from_numpy(sc).to(DEV),
                        torch.tensor(lens, dtype=torch.int32, device=DEV), k,
                        stride, idx, cnt, ws, ws_zeroed=zeroed)
        torch.cuda.synchronize()
        ridx, rcnt = oracle.topk(sc, lens, k)
        np.testing.assert_array_equal(cnt.cpu().numpy(), rcnt)
        np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
        assert not _hist_words(ws, r).any(), "histograms left nonzero"


def test_fused_topk_reuses_a_zeroed_workspace():
    """sparse_index_topk flagged on a zero-filled workspace, several layers
    in turn: identical to the unflagged call on a fresh workspace."""
    import top_sparse_decode_amd as tsd
    cfg = tsd_synth.config(QSA, B=3, lens=(70000, 3000, 33333), top_k=2048,
                           chunks=4, seed=402)
    B, k = cfg.B, cfg.top_k
    ws = None
    for layer in range(3):
        wl = tsd_synth.make(cfg, DEV, layer=layer)
        stride = wl["page_table"].shape[1] * 64
        outs = []
        for zeroed in (True, False):
            S = torch.empty((B, stride), device=DEV)
            rl = torch.empty(B, dtype=torch.int32, device=DEV)
            idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
            cnt = torch.empty(B, dtype=torch.int32, device=DEV)
            nbytes = tsd.topk_select_workspace_bytes(B, stride, k)
            if zeroed and ws is None:
                ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
            w = ws if zeroed else torch.full((nbytes,), 0x5C, dtype=torch.uint8,
                                             device=DEV)
            tsd.sparse_index_topk("qsa", S, wl["page_table"], wl["seq_lens"],
                                  wl["num_pages"], k, idx, cnt, w, rl,
                                  index_q=wl["index_q"], index_w=wl["index_w"],
                                  index_k_pool=wl["index_k"], ws_zeroed=zeroed)
            torch.cuda.synchronize()
            outs.append((S.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()))
            assert not _hist_words(w, B).any()
        np.testing.assert_array_equal(outs[0][1], outs[1][1])
        np.testing.assert_array_equal(outs[0][2], outs[1][2])
        lens = wl["seq_lens"].cpu().numpy()
        check_topk_identical(outs[0][0], lens, k, outs[0][1], outs[0][2])


@pytest.mark.parametrize("stride", [10000, 70000])
def test_topk_special_rows_bit_exact(stride):
    """Degenerate rows on the one-workgroup path (rows of at most 32,768
    entries) and, with the same rows in a wider buffer, the chunked path."""
    rng = np.random.default_rng(5)
    k = 300
    lens = [0, 1, 299, 300, 301, 10000, 10000, 10000, 10000, 9999, 5000]
    s = np.full((len(lens), stride), np.nan, dtype=np.float32)
    s[:, :10000] = rng.normal(size=(len(lens), 10000)).astype(np.float32)
    s[5, :10000] = 3.25                          # all equal
    s[6, :10000] = rng.choice([-0.0, 0.0], size=10000)  # signed zeros only
    s[7, :10000:7] = np.inf
    s[7, 1:10000:7] = -np.inf
    s[8, :10000] = rng.integers(0, 4, size=10000).astype(np.float32)  # ties
    s[9, :10000] = -np.abs(s[9, :10000])         # all negative
    s[10, :5000] = np.linspace(1, 0, 5000)       # strictly decreasing
    gidx, gcnt = _topk_gpu(s, lens, k)
    ridx, rcnt = oracle.topk(s, lens, k)
    np.testing.assert_array_equal(gcnt, rcnt)
    np.testing.assert_array_equal(gidx, ridx)
    assert (gidx[5, :300] == np.arange(300)).all()
    assert (gidx[0] == -1).all() and gcnt[0] == 0


@pytest.mark.parametrize("max_len,k", [(300, 1), (4096, 256), (4097, 4096),
                                       (8192, 2048), (8193, 300), (16385, 1024),
                                       (16384, 2048), (20224, 1024), (23000, 512),
                                       (28000, 3000), (32768, 4096), (32769, 1),
                                       (60032, 3000)])
def test_topk_one_workgroup_rows(max_len, k):
    """Rows of at most 32,768 entries (the whole row in one workgroup's
    registers), across the register templates and their boundaries, and
    just past them on the chunked path: normal values, three levels (ties
    at the threshold), rows of n = k, k + 1, a ragged tail and an empty row,
    against the oracle."""
    rng = np.random.default_rng(max_len * 7 + k)
    rows = 6
    s = np.empty((rows, max_len), np.float32)
    s[0] = rng.normal(size=max_len)
    s[1] = (rng.integers(0, 3, size=max_len) / 3).astype(np.float32)
    s[2] = rng.normal(size=max_len)
    s[3] = rng.normal(size=max_len)
    s[4] = np.float32(1.0)
    s[5] = rng.normal(size=max_len)
    lens = [max_len, max_len - 1, min(k, max_len), min(k + 1, max_len),
            max(1, max_len // 3 + 17), 0]
    gidx, gcnt = _topk_gpu(s, lens, k)
    ridx, rcnt = oracle.topk(s, lens, k)
    np.testing.assert_array_equal(gcnt, rcnt)
    np.testing.assert_array_equal(gidx, ridx)


def test_topk_filter_runs_several_passes_per_workgroup():
    """100 rows in a buffer of 1,048,576 entries: the filter's launch would
    exceed 1,024 workgroups, so each workgroup walks 8 passes of 4 chunks
    (two passes' scores in flight); rows of 30,000-150,000 entries end
    inside a workgroup's passes, one row fills the buffer. Ties at the
    threshold from 5,000 levels. Against the oracle."""
    rng = np.random.default_rng(311)
    rows, L, k = 100, 1 << 20, 2048
    lens = rng.integers(30000, 150000, size=rows).tolist()
    lens[37] = L
    s = np.full((rows, L), np.nan, np.float32)
    for r, n in enumerate(lens):
        s[r, :n] = rng.integers(0, 5000, size=n) / 5000
    gidx, gcnt = _topk_gpu(s, lens, k)
    ridx, rcnt = oracle.topk(np.nan_to_num(s, nan=0.0), lens, k)
    np.testing.assert_array_equal(gcnt, rcnt)
    np.testing.assert_array_equal(gidx, ridx)


@pytest.mark.parametrize("c", [10000, 16388, 16389, 19000])
def test_topk_one_workgroup_crowded_digit1_bin(c):
    """One-workgroup rows whose k-th largest key lies in a digit-1 bin of
    thousands of keys: c entries tie at 1.0 (one digit-1 bin) and the rest
    lie above it (c = 10,000 leaves the k-th largest among them); the
    second row's length cuts three entries. Against the oracle."""
    rng = np.random.default_rng(c)
    L, k = 20000, 4000
    rows = 2
    s = np.empty((rows, L), np.float32)
    for r in range(rows):
        s[r] = 2.0 + rng.random(L).astype(np.float32)
        s[r, rng.permutation(L)[:c]] = 1.0
    lens = [L, L - 3]
    gidx, gcnt = _topk_gpu(s, lens, k)
    ridx, rcnt = oracle.topk(s, lens, k)
    np.testing.assert_array_equal(gcnt, rcnt)
    np.testing.assert_array_equal(gidx, ridx)


def test_topk_one_workgroup_rows_clear_an_unflagged_workspace():
    """The one-workgroup path reads no workspace, yet an unflagged call still
    leaves the histogram words zero for the flagged calls that follow."""
    import top_sparse_decode_amd as tsd
    rng = np.random.default_rng(31)
    rows, max_len, k = 4, 20000, 1024
    s = rng.normal(size=(rows, max_len)).astype(np.float32)
    lens = [20000, 19999, 5000, 1024]
    ws = torch.full((tsd.topk_select_workspace_bytes(rows, max_len, k),), 0x3C,
                    dtype=torch.uint8, device=DEV)
    ridx, rcnt = oracle.topk(s, lens, k)
    for zeroed in (False, True):
        idx = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
        cnt = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
        tsd.topk_select(torch.from_numpy(s).to(DEV),
                        torch.tensor(lens, dtype=torch.int32, device=DEV), k,
                        max_len, idx, cnt, ws, ws_zeroed=zeroed)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(cnt.cpu().numpy(), rcnt)
        np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
        assert not _hist_words(ws, rows).any()


@pytest.mark.parametrize("n,k,levels", [(50000, 3000, 3), (262144, 2048, 50),
                                        (70000, 4096, 1_000_000)])
def test_topk_large_rows_with_ties(n, k, levels):
    rng = np.random.default_rng(n)
    s = (rng.integers(0, levels, size=(3, n)) / levels).astype(np.float32)
    lens = [n, n - 1, n // 3]
    gidx, gcnt = _topk_gpu(s, lens, k)
    ridx, rcnt = oracle.topk(s, lens, k)
    np.testing.assert_array_equal(gcnt, rcnt)
    np.testing.assert_array_equal(gidx, ridx)


def test_topk_rows_past_one_million_entries():
    """Rows of more than 1,048,576 entries (more chunks than the resolve's
    blind reads cover): the staged and bitmap paths, against the oracle."""
    rng = np.random.default_rng(2200000)
    n = 2_200_000
    s = np.empty((3, n), np.float32)
    s[0] = rng.normal(size=n)
    s[1] = (rng.integers(0, 30, size=n) / 30).astype(np.float32)  # heavy ties
    s[2] = rng.normal(size=n)
    s[2, 1_500_000:1_504_096] += 30.0   # the top values in one chunk
    lens = [n, n - 3, 1_200_001]
    for k in (2048, 4096):
        gidx, gcnt = _topk_gpu(s, lens, k)
        ridx, rcnt = oracle.topk(s, lens, k)
        np.testing.assert_array_equal(gcnt, rcnt)
        np.testing.assert_array_equal(gidx, ridx)


def test_topk_ties_at_threshold_and_one_overflowing_chunk():
    # row 0: a few ties planted at the k-th largest value of a normal row,
    # more than are kept (every chunk list fits); row 1: one 4,096-element
    # chunk holds 700 of the largest values (its list overflows and is read
    # raw); row 2: 6,000 survivors spread evenly (a large fits-all case)
    rng = np.random.default_rng(17)
    n, k = 262144, 2048
    s = rng.normal(size=(3, n)).astype(np.float32)
    t = np.sort(s[0])[::-1][k - 1]
    s[0, rng.choice(n, size=40, replace=False)] = t
    s[1, 5 * 4096:5 * 4096 + 700] = 10.0 + rng.random(700).astype(np.float32)
    s[2] = np.where(rng.random(n) < 6000 / n, 5.0, s[2]).astype(np.float32)
    lens = [n, n, n]
    gidx, gcnt = _topk_gpu(s, lens, k)
    ridx, rcnt = oracle.topk(s, lens, k)
    np.testing.assert_array_equal(gcnt, rcnt)
    np.testing.assert_array_equal(gidx, ridx)


# --------------------------------------------------- sharded top-k merge
@pytest.mark.parametrize("W", [1, 3, 4, 8])
def test_merge_sharded_matches_unsharded_topk(W):
    import top_sparse_decode_amd as tsd
    rng = np.random.default_rng(40 + W)
    ns = [70000, 4096 * 3 + 17, 64 * W - 5, 0, 2500, 150000]
    k = 2048
    rows = len(ns)
    full = np.full((rows, max(ns)), np.nan, np.float32)
    for r, n in enumerate(ns):
        levels = [1000, 7, 50, 1, 3, 100000][r]
        full[r, :n] = rng.integers(0, levels, size=n) / levels
        full[r, :n][rng.random(n) < 0.02] = -0.0
    # shard-local score rows: shard w holds the tokens of pages p % W == w
    orders = [oracle.shard_row_order(n, W) for n in ns]
    L = max(1, max(len(o) for ord_ in orders for o in ord_))
    S = np.full((W, rows, L), np.nan, np.float32)
    lens = np.zeros((W, rows), np.int32)
    for r, ord_ in enumerate(orders):
        for w, o in enumerate(ord_):
            S[w, r, :len(o)] = full[r, o]
            lens[w, r] = len(o)
    Sg = torch.from_numpy(S).to(DEV)
    lg = torch.from_numpy(lens).to(DEV)
    il, cl = gpu_topk_stack(Sg, lg, k)
    idx = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    tsd.topk_merge_sharded(Sg, il, cl, k, idx, cnt)
    torch.cuda.synchronize()
    ridx, rcnt = oracle.topk(np.nan_to_num(full, nan=0.0), ns, k)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rcnt)
    np.testing.assert_array_equal(idx.cpu().numpy(), ridx)
    # the oracle merge of the GPU's shard lists agrees as well
    midx, _ = oracle.topk_merge_sharded(S, il.cpu().numpy(), cl.cpu().numpy(), k)
    np.testing.assert_array_equal(idx.cpu().numpy(), midx)


def test_merge_sharded_sixteen_shards_and_unordered_lists():
    """W = 16 shards of k = kl = 1,024 candidates (the most a row takes),
    with ties: the merge of the shard top-k lists equals the oracle merge;
    the same lists with their entries shuffled (not ascending, as
    topk_select never writes them) give the same result."""
    import top_sparse_decode_amd as tsd
    rng = np.random.default_rng(47)
    W, rows, L, k = 16, 2, 6000, 1024
    S = (rng.integers(0, 300, size=(W, rows, L)) / 300).astype(np.float32)
    lens = np.full((W, rows), L, np.int32)
    lens[3, 1] = 700  # a short shard: fewer than k candidates
    Sg = torch.from_numpy(S).to(DEV)
    il, cl = gpu_topk_stack(Sg, torch.from_numpy(lens).to(DEV), k)
    midx, mcnt = oracle.topk_merge_sharded(S, il.cpu().numpy(), cl.cpu().numpy(), k)
    for shuffle in (False, True):
        if shuffle:
            g = torch.Generator(device="cpu").manual_seed(5)
            ilh = il.cpu()
            for w in range(W):
                for r in range(rows):
                    c = int(cl[w, r])
                    ilh[w, r, :c] = ilh[w, r, :c][torch.randperm(c, generator=g)]
            il = ilh.to(DEV)
        idx = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
        cnt = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
        tsd.topk_merge_sharded(Sg, il, cl, k, idx, cnt)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(cnt.cpu().numpy(), mcnt)
        np.testing.assert_array_equal(idx.cpu().numpy(), midx)


def test_merge_sharded_rows_past_one_bitmap_segment():
    """Four shards of 400,000 tokens: a row's global tokens run to 1.6M,
    past the merge's 1,048,576-token output bitmap, so its kept tokens are
    written over two segments; the result equals the oracle merge."""
    import top_sparse_decode_amd as tsd
    rng = np.random.default_rng(53)
    W, rows, L, k = 4, 2, 400000, 2048
    S = rng.standard_normal((W, rows, L)).astype(np.float32)
    lens = np.full((W, rows), L, np.int32)
    lens[2, 1] = 300000
    Sg = torch.from_numpy(S).to(DEV)
    il, cl = gpu_topk_stack(Sg, torch.from_numpy(lens).to(DEV), k)
    midx, mcnt = oracle.topk_merge_sharded(S, il.cpu().numpy(), cl.cpu().numpy(), k)
    assert (midx >= 1 << 20).any() and ((midx >= 0) & (midx < 1 << 20)).any()
    idx = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    tsd.topk_merge_sharded(Sg, il, cl, k, idx, cnt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(cnt.cpu().numpy(), mcnt)
    np.testing.assert_array_equal(idx.cpu().numpy(), midx)


def test_merge_sharded_short_lists_and_bad_entries():
    import top_sparse_decode_amd as tsd
    # hand-made candidate lists: counts below kl, -1 and out-of-range
    # entries are ignored; k above the number of candidates pads with -1
    W, rows, stride, kl, k = 2, 1, 128, 4, 6
    S = torch.zeros((W, rows, stride), device=DEV)
    S[0, 0, :4] = torch.tensor([1.0, 9.0, 3.0, 9.0])
    S[1, 0, :4] = torch.tensor([9.0, 2.0, 5.0, 4.0])
    il = torch.tensor([[[1, 3, 2, 0]], [[0, -1, 500, 3]]], dtype=torch.int32,
                      device=DEV)
    cl = torch.tensor([[3], [4]], dtype=torch.int32, device=DEV)
    idx = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    tsd.topk_merge_sharded(S, il, cl, k, idx, cnt)
    torch.cuda.synchronize()
    # shard 0 local 1, 3, 2 -> global 1, 3, 2; shard 1 local 0, 3 -> 64, 67
    assert cnt.item() == 5
    assert idx[0].tolist() == [1, 2, 3, 64, 67, -1]
    out3 = torch.empty((rows, 3), dtype=torch.int32, device=DEV)
    tsd.topk_merge_sharded(S, il, cl, 3, out3, cnt)
    torch.cuda.synchronize()
    assert out3[0].tolist() == [1, 3, 64]  # 9, 9, 9: lowest global tokens


def test_sharded_qsa_pipeline_equals_unsharded():
    """Each shard scores and selects over its own pages; the merge equals the
    unsharded sparse_index_topk bit for bit."""
    cfg = tsd_synth.config(QSA, B=2, lens=(70000, 33333), top_k=2048,
                           chunks=8, seed=160)
    wl = tsd_synth.make(cfg, DEV)
    bufs = _run(wl)
    idx, cnt, _, lens = sharded_qsa_select(wl, 4, cfg.top_k)
    torch.cuda.synchronize()
    assert lens.sum(0).tolist() == list(cfg.lens)
    assert torch.equal(idx, bufs.idx.view(cfg.B, cfg.top_k))
    assert torch.equal(cnt, bufs.count.view(cfg.B))


# ------------------------------------------- block-compressed QSA select
@pytest.mark.parametrize("Bs,lens", [(1, (700, 64)), (2, (130, 1)),
                                     (4, (9000, 1000, 3)), (8, (3000, 511)),
                                     (16, (5000, 4097)), (32, (10000, 33)),
                                     (64, (20000, 65))])
def test_index_k_compress_matches_oracle(Bs, lens):
    import top_sparse_decode_amd as tsd
    cfg = tsd_synth.config(QSA, B=len(lens), lens=lens, seed=190 + Bs)
    wl = tsd_synth.make(cfg, DEV)
    lay = tsd_synth.compressed_layout(wl, Bs)
    lay["ck_pool"].fill_(0x11)
    from_block = torch.tensor([i % 2 for i in range(len(lens))],
                              dtype=torch.int32, device=DEV)
    max_blocks = int(lay["block_lens"].max())
    h = tsd_synth.to_host(wl)
    ref = oracle.index_k_compress(h["index_k"], h["page_table"], h["num_pages"],
                                  h["seq_lens"], from_block.cpu().numpy(),
                                  lay["cpage_table"].cpu().numpy(),
                                  lay["num_cpages"], lay["ck_pool"].cpu().numpy(),
                                  Bs)
    tsd.index_k_compress(wl["index_k"], wl["page_table"], wl["num_pages"],
                         wl["seq_lens"], lay["ck_pool"], lay["cpage_table"],
                         lay["num_cpages"], Bs, max_blocks, from_block)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lay["ck_pool"].cpu().numpy(), ref)


@pytest.mark.parametrize("Bs", [1, 4, 64])
def test_index_k_compress_last_block_per_step(Bs):
    """The per-step update: one block per request, the one holding the last
    token (max_blocks = 1), over a pool holding other values."""
    import top_sparse_decode_amd as tsd
    lens = (4097, 64, 1, 30001)
    cfg = tsd_synth.config(QSA, B=len(lens), lens=lens, seed=300 + Bs)
    wl = tsd_synth.make(cfg, DEV)
    lay = tsd_synth.compressed_layout(wl, Bs)
    lay["ck_pool"].fill_(0x5a)
    last = (lay["block_lens"] - 1).clamp(min=0)
    h = tsd_synth.to_host(wl)
    ref = oracle.index_k_compress(h["index_k"], h["page_table"], h["num_pages"],
                                  h["seq_lens"], last.cpu().numpy(),
                                  lay["cpage_table"].cpu().numpy(),
                                  lay["num_cpages"], lay["ck_pool"].cpu().numpy(),
                                  Bs)
    tsd.index_k_compress(wl["index_k"], wl["page_table"], wl["num_pages"],
                         wl["seq_lens"], lay["ck_pool"], lay["cpage_table"],
                         lay["num_cpages"], Bs, 1, last)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(lay["ck_pool"].cpu().numpy(), ref)


def test_expand_blocks_matches_oracle():
    import top_sparse_decode_amd as tsd
    rng = np.random.default_rng(7)
    rows, kb = 6, 512
    for Bs in (1, 4, 64):
        lens = rng.integers(0, 300000, rows).astype(np.int32)
        lens[0], lens[1] = 0, 5
        sel = np.full((rows, kb), -1, np.int32)
        cnt = np.zeros(rows, np.int32)
        for r in range(rows):
            nb = -(-int(lens[r]) // Bs)
            c = min(kb, nb, int(rng.integers(0, kb + 1)))
            sel[r, :c] = np.sort(rng.choice(max(nb, 1), size=c, replace=False))
            cnt[r] = c
        cnt[2] = kb + 5  # clamped to kb
        for kt in (2048, 4096, 100):
            ref, rc = oracle.expand_blocks(sel, np.minimum(cnt, kb), Bs, lens, kt)
            tok = torch.full((rows, kt), -7, dtype=torch.int32, device=DEV)
            tc = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
            tsd.expand_blocks(torch.from_numpy(sel).to(DEV),
                              torch.from_numpy(cnt).to(DEV), Bs,
                              torch.from_numpy(lens).to(DEV), tok, tc)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(tok.cpu().numpy(), ref)
            np.testing.assert_array_equal(tc.cpu().numpy(), rc)


def _block_select(wl, Bs, kb):
    """Compress every block, score and select blocks with the fused call,
    expand to tokens. Returns (layout, block scores, block idx, block count,
    token idx [B, 1, kb*Bs], token count [B, 1])."""
    import top_sparse_decode_amd as tsd
    B = wl["B"]
    lay = tsd_synth.compressed_layout(wl, Bs)
    tsd.index_k_compress(wl["index_k"], wl["page_table"], wl["num_pages"],
                         wl["seq_lens"], lay["ck_pool"], lay["cpage_table"],
                         lay["num_cpages"], Bs, int(lay["block_lens"].max()))
    stride = lay["cpage_table"].shape[1] * 64
    scores = torch.full((B, stride), float("nan"), device=DEV)
    rl = torch.empty(B, dtype=torch.int32, device=DEV)
    bidx = torch.empty((B, kb), dtype=torch.int32, device=DEV)
    bcnt = torch.empty(B, dtype=torch.int32, device=DEV)
    ws = torch.empty(tsd.topk_select_workspace_bytes(B, stride, kb),
                     dtype=torch.uint8, device=DEV)
    tsd.sparse_index_topk("qsa", scores, lay["cpage_table"], lay["block_lens"],
                          lay["num_cpages"], kb, bidx, bcnt, ws, rl,
                          index_q=wl["index_q"], index_w=wl["index_w"],
                          index_k_pool=lay["ck_pool"])
    tok = torch.empty((B, 1, kb * Bs), dtype=torch.int32, device=DEV)
    tcnt = torch.empty((B, 1), dtype=torch.int32, device=DEV)
    tsd.expand_blocks(bidx, bcnt, Bs, wl["seq_lens"], tok.view(B, -1),
                      tcnt.view(B))
    return lay, scores, rl, bidx, bcnt, tok, tcnt


@pytest.mark.parametrize("Bs,lens,kb", [(4, (30000, 3000, 100), 512),
                                        (16, (65536, 2000), 128)])
def test_block_compressed_decode_path(Bs, lens, kb):
    """Compressed keys, block scores, block top-k, expansion and the sparse
    attention over the expanded tokens, each against the oracle."""
    import top_sparse_decode_amd as tsd
    cfg = tsd_synth.config(QSA, B=len(lens), lens=lens, top_k=kb * Bs,
                           chunks=8, seed=200 + Bs)
    wl = tsd_synth.make(cfg, DEV)
    lay, scores, rl, bidx, bcnt, tok, tcnt = _block_select(wl, Bs, kb)
    B, kt = cfg.B, kb * Bs
    o = torch.empty((B, cfg.H_q, cfg.chunks, 128), device=DEV)
    lse = torch.empty((B, cfg.H_q, cfg.chunks), device=DEV)
    tsd.sparse_gqa_decode(wl["q"], wl["k_pool"], wl["v_pool"], wl["page_table"],
                          wl["seq_lens"], wl["num_pages"], tok, tcnt, cfg.chunks,
                          o, lse, k_scale=wl["k_scale"], v_scale=wl["v_scale"])
    torch.cuda.synchronize()
    h = tsd_synth.to_host(wl)
    ck = oracle.index_k_compress(h["index_k"], h["page_table"], h["num_pages"],
                                 h["seq_lens"], np.zeros(B, np.int32),
                                 lay["cpage_table"].cpu().numpy(),
                                 lay["num_cpages"],
                                 np.zeros_like(lay["ck_pool"].cpu().numpy()), Bs)
    np.testing.assert_array_equal(lay["ck_pool"].cpu().numpy(), ck)
    blens = lay["block_lens"].cpu().numpy()
    np.testing.assert_array_equal(rl.cpu().numpy(), blens)
    ref_s = oracle.qsa_scores(h["index_q"], h["index_w"], ck,
                              lay["cpage_table"].cpu().numpy(), blens,
                              lay["num_cpages"],
                              score_stride=scores.shape[1])
    gs = scores.cpu().numpy()
    check_scores(gs, ref_s, blens, score_tol("qsa"))
    check_topk_identical(gs, blens, kb, bidx.cpu().numpy(), bcnt.cpu().numpy())
    rtok, rcnt = oracle.expand_blocks(bidx.cpu().numpy(), bcnt.cpu().numpy(), Bs,
                                      h["seq_lens"], kt)
    np.testing.assert_array_equal(tok.view(B, kt).cpu().numpy(), rtok)
    np.testing.assert_array_equal(tcnt.view(B).cpu().numpy(), rcnt)
    check_attention_on(h, tok.cpu().numpy(), tcnt.cpu().numpy(), cfg.chunks,
                       o.cpu().numpy(), lse.cpu().numpy(), out_tol(cfg.kv_enc))


@pytest.mark.parametrize("name,Bs,lens,kb,C", [
    (QSA, 4, (30000, 4097, 100, 6), 512, 7),
    (QSA, 16, (65536, 2000, 17), 128, 16),
    (QSA, 64, (5000, 64, 65), 16, 5),
    (DS8B, 8, (9000, 1001), 200, 4),
])
def test_block_index_attention_equals_expanded_tokens(name, Bs, lens, kb, C):
    """sparse_gqa_decode on block indices (idx_block = Bs) gives exactly the
    result of expand_blocks followed by attention over those tokens: full
    and short selections, with the partial last block selected or not, for
    a shared (FP8) and a per-KV-head (BF16) selection."""
    import top_sparse_decode_amd as tsd
    cfg = tsd_synth.config(name, B=len(lens), lens=lens, top_k=kb * Bs,
                           chunks=C, seed=230 + Bs)
    wl = tsd_synth.make(cfg, DEV)
    B = cfg.B
    H_sel = 1 if cfg.mode == "qsa" else cfg.H_kv
    g = torch.Generator().manual_seed(231)
    sel = torch.full((B, H_sel, kb), -1, dtype=torch.int32)
    cnt = torch.zeros((B, H_sel), dtype=torch.int32)
    for b, n in enumerate(lens):
        nb = (n + Bs - 1) // Bs
        for hs in range(H_sel):
            c = min(kb, nb) if (b + hs) % 3 else max(1, min(kb, nb) // 2)
            pick = torch.randperm(nb, generator=g)[:c]
            if (b + hs) % 2 == 0 and nb - 1 not in pick.tolist():
                pick[0] = nb - 1  # the (possibly partial) last block
            sel[b, hs, :c] = pick.sort().values.to(torch.int32)
            cnt[b, hs] = c
    sel_d, cnt_d = sel.to(DEV), cnt.to(DEV)
    kt = kb * Bs
    tok = torch.empty((B, H_sel, kt), dtype=torch.int32, device=DEV)
    tcnt = torch.empty((B, H_sel), dtype=torch.int32, device=DEV)
    tsd.expand_blocks(sel_d.view(B * H_sel, kb), cnt_d.view(-1), Bs,
                      wl["seq_lens"].repeat_interleave(H_sel),
                      tok.view(B * H_sel, kt), tcnt.view(-1))
    outs = []
    for ix, cn, blk in ((tok, tcnt, 0), (sel_d, cnt_d, Bs)):
        o = torch.full((B, cfg.H_q, C, 128), float("nan"), device=DEV)
        lse = torch.full((B, cfg.H_q, C), float("nan"), device=DEV)
        tsd.sparse_gqa_decode(wl["q"], wl["k_pool"], wl["v_pool"],
                              wl["page_table"], wl["seq_lens"],
                              wl["num_pages"], ix, cn, C, o, lse,
                              k_scale=wl.get("k_scale"),
                              v_scale=wl.get("v_scale"), idx_block=blk)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])
    # the expansion's token counts are the block selection's token lengths
    nb_tok = [[int(cnt[b, hs]) * Bs
               - max(0, (int(sel[b, hs, cnt[b, hs] - 1]) + 1) * Bs - lens[b])
               for hs in range(H_sel)] for b in range(B)]
    np.testing.assert_array_equal(tcnt.cpu().numpy(), np.array(nb_tok))


# -------------------------------------------------- sparse-decode threshold
@pytest.mark.parametrize("name,lens,dense_len", [
    ("ds_llama31_8b_b3_l60000", (300, 5000, 1000), 1000),
    (QSA, (700, 9000, 2048, 64), 2048),
])
def test_dense_threshold_requests_attend_to_every_token(name, lens, dense_len):
    """Requests no longer than dense_len attend densely (selection = every
    token, through the chunked kernel); the others keep their top-k."""
    cfg = tsd_synth.config(name, B=len(lens), lens=lens, top_k=256, chunks=5,
                           seed=180)
    wl = tsd_synth.make(cfg, DEV)
    wl["dense_len"] = dense_len
    bufs = _run(wl)
    h = tsd_synth.to_host(wl)
    H_sel = bufs.H_sel
    kmax = max(max(lens), cfg.top_k)
    idx = np.full((cfg.B, H_sel, kmax), -1, np.int32)
    cnt = np.zeros((cfg.B, H_sel), np.int32)
    gidx = bufs.idx.view(cfg.B, H_sel, cfg.top_k).cpu().numpy()
    gcnt = bufs.count.view(cfg.B, H_sel).cpu().numpy()
    for b, n in enumerate(lens):
        if n <= dense_len:
            idx[b, :, :n] = np.arange(n)
            cnt[b] = n
        else:
            idx[b, :, :cfg.top_k] = gidx[b]
            cnt[b] = gcnt[b]
    check_attention_on(h, idx, cnt, cfg.chunks, bufs.o_part.cpu().numpy(),
                       bufs.lse_part.cpu().numpy(), out_tol(cfg.kv_enc))
    check_merge(bufs.o_part.cpu().numpy(), bufs.lse_part.cpu().numpy(),
                bufs.out.cpu().numpy(), bufs.out_lse.cpu().numpy())
    # a dense request's idx row may be loaded but is never used: garbage
    # entries and counts there leave every partial bit for bit unchanged
    import top_sparse_decode_amd.step as step
    o0, l0 = bufs.o_part.clone(), bufs.lse_part.clone()
    iv = bufs.idx.view(cfg.B, H_sel, cfg.top_k)
    cv = bufs.count.view(cfg.B, H_sel)
    for b, n in enumerate(lens):
        if n <= dense_len:
            iv[b] = torch.randint(-2 ** 31, 2 ** 31 - 1, iv[b].shape,
                                  dtype=torch.int32, device=DEV)
            cv[b] = 123457
    step.attend(wl, bufs)
    torch.cuda.synchronize()
    assert torch.equal(bufs.o_part, o0)
    assert torch.equal(bufs.lse_part, l0)


# ------------------------------------------------------------ cache append
def _u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_append_fp8_kv_and_index_match_oracle():
    import top_sparse_decode_amd as tsd
    g = torch.Generator(device="cpu").manual_seed(70)
    B, H, D, P, NP, max_new = 3, 4, 128, 6, 40, 150
    pt = torch.randperm(NP, generator=g)[:B * P].view(B, P).to(torch.int32)
    pt[2, 4] = NP + 3  # a bad page id: its tokens are skipped
    positions = torch.tensor([0, 70, 250], dtype=torch.int32)
    n_new = torch.tensor([150, 1, 140], dtype=torch.int32)  # 250+140 > 6*64
    codes = torch.randint(0, 0x7E, (NP * 64, H, D), generator=g).to(torch.uint8)
    codes |= (torch.rand(codes.shape, generator=g) < 0.5).to(torch.uint8) << 7
    kp, vp = codes.clone(), codes.flip(0).contiguous()
    ks = torch.rand(NP, generator=g) * 0.05 + 1e-3
    vs = torch.rand(NP, generator=g) * 0.05 + 1e-3
    kn = (torch.randn((B, max_new, H, D), generator=g) * 5).to(torch.bfloat16)
    vn = (torch.randn((B, max_new, H, D), generator=g) * 5).to(torch.bfloat16)
    ikp = torch.randint(0, 0x7E, (NP * 64, 128), generator=g).to(torch.uint8)
    ikn = torch.randn((B, max_new, 128), generator=g) * 100
    ref = oracle.kv_append(pt.numpy(), NP, positions.numpy(), n_new.numpy(),
                           max_new, k_new=_u16(kn), v_new=_u16(vn),
                           k_pool=kp.numpy(), v_pool=vp.numpy(),
                           kv_enc="fp8_e4m3", k_scale=ks.numpy(),
                           v_scale=vs.numpy(), index_k_new=ikn.numpy(),
                           index_enc="f32", index_k_pool=ikp.numpy())
    d = {n: t.to(DEV) for n, t in dict(pt=pt, pos=positions, n=n_new, kp=kp,
                                       vp=vp, ks=ks, vs=vs, kn=kn, vn=vn,
                                       ikp=ikp, ikn=ikn).items()}
    tsd.kv_append(d["pt"], NP, d["pos"], d["n"], max_new, k_new=d["kn"],
                  v_new=d["vn"], k_pool=d["kp"], v_pool=d["vp"],
                  k_scale=d["ks"], v_scale=d["vs"], index_k_new=d["ikn"],
                  index_k_pool=d["ikp"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d["ks"].cpu().numpy(), ref["k_scale"])
    np.testing.assert_array_equal(d["vs"].cpu().numpy(), ref["v_scale"])
    np.testing.assert_array_equal(d["kp"].cpu().numpy(), ref["k_pool"])
    np.testing.assert_array_equal(d["vp"].cpu().numpy(), ref["v_pool"])
    np.testing.assert_array_equal(d["ikp"].cpu().numpy(), ref["index_k_pool"])
    # request 1 appends at 70 onto a page begun at 64: its scale is kept
    assert d["ks"][pt[1, 1]].item() == ks[pt[1, 1]].item()


def test_append_16bit_rows_and_label_match_oracle():
    import top_sparse_decode_amd as tsd
    g = torch.Generator(device="cpu").manual_seed(71)
    B, H, D, P, NP, r, max_new = 2, 8, 128, 5, 12, 16, 70
    pt = torch.randperm(NP, generator=g)[:B * P].view(B, P).to(torch.int32)
    pt[0, 2] = -1
    positions = torch.tensor([100, 5], dtype=torch.int32)
    n_new = torch.tensor([70, 64], dtype=torch.int32)
    ch = torch.stack([torch.randperm(D, generator=g)[:r] for _ in range(H)]).to(torch.int32)
    ch[3, 0], ch[5, 7] = -1, 200  # outside [0, D): stores 0
    kp = torch.randn((NP * 64, H, D), generator=g).to(torch.float16)
    vp = torch.randn((NP * 64, H, D), generator=g).to(torch.float16)
    lp = torch.randn((NP * 64, H, r), generator=g).to(torch.float16)
    kn = torch.randn((B, max_new, H, D), generator=g).to(torch.float16)
    vn = torch.randn((B, max_new, H, D), generator=g).to(torch.float16)
    ref = oracle.kv_append(pt.numpy(), NP, positions.numpy(), n_new.numpy(),
                           max_new, k_new=_u16(kn), v_new=_u16(vn),
                           new_enc="fp16", k_pool=_u16(kp), v_pool=_u16(vp),
                           kv_enc="fp16", channel_idx=ch.numpy(),
                           label_pool=_u16(lp))
    d = {n: t.to(DEV) for n, t in dict(pt=pt, pos=positions, n=n_new, kp=kp,
                                       vp=vp, lp=lp, kn=kn, vn=vn, ch=ch).items()}
    tsd.kv_append(d["pt"], NP, d["pos"], d["n"], max_new, k_new=d["kn"],
                  v_new=d["vn"], k_pool=d["kp"], v_pool=d["vp"],
                  channel_idx=d["ch"], label_pool=d["lp"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_u16(d["kp"]), ref["k_pool"])
    np.testing.assert_array_equal(_u16(d["vp"]), ref["v_pool"])
    np.testing.assert_array_equal(_u16(d["lp"]), ref["label_pool"])


def test_append_index_fp8_encode_every_case():
    """The gfx950 converter behind kv_append gives the oracle's code for
    every finite E4M3 value, every midpoint and its neighbours, the
    subnormal range, signed zeros and out-of-range magnitudes."""
    import top_sparse_decode_amd as tsd
    vals = [oracle.decode_fp8_e4m3(c) for c in range(256) if c & 0x7F != 0x7F]
    pos = [oracle.decode_fp8_e4m3(c) for c in range(0x7F)]
    for c in range(0x7E):
        mid = (pos[c] + pos[c + 1]) / 2
        for m in (mid, np.nextafter(np.float32(mid), np.float32(0)),
                  np.nextafter(np.float32(mid), np.float32(1e9))):
            vals += [float(m), -float(m)]
    vals += [448.0, 463.9, 464.0, 480.0, 1e6, -1e30, 0.0, -0.0, 2.0 ** -12,
             -2.0 ** -11, 1e-30, 3e38]
    x = np.array(vals, np.float32)
    n = -(-len(x) // 128)
    xs = np.zeros(n * 128, np.float32)
    xs[:len(x)] = x
    ikn = torch.from_numpy(xs.reshape(1, n, 128))
    pt = torch.arange((n + 63) // 64, dtype=torch.int32)[None]
    ikp = torch.zeros((pt.shape[1] * 64, 128), dtype=torch.uint8)
    ref = oracle.kv_append(pt.numpy(), pt.shape[1], [0], [n], n,
                           index_k_new=ikn.numpy(), index_enc="f32",
                           index_k_pool=ikp.numpy())
    gi = ikp.to(DEV)
    tsd.kv_append(pt.to(DEV), pt.shape[1], torch.zeros(1, dtype=torch.int32, device=DEV),
                  torch.tensor([n], dtype=torch.int32, device=DEV), n,
                  index_k_new=ikn.to(DEV), index_k_pool=gi)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gi.cpu().numpy(), ref["index_k_pool"])


def test_topk_row_lens_clamped_to_max_len():
    rng = np.random.default_rng(9)
    s = rng.normal(size=(2, 5000)).astype(np.float32)
    gidx, gcnt = _topk_gpu(s, [100000, -5], 50, max_len=4000)
    ridx, rcnt = oracle.topk(s, [4000, 0], 50)
    np.testing.assert_array_equal(gidx, ridx)
    np.testing.assert_array_equal(gcnt, rcnt)


# ----------------------------------------------------------- merge and misc
@pytest.mark.parametrize("C,D", [(64, 128), (16, 128), (5, 128), (17, 128),
                                 (24, 100), (33, 200), (63, 128)])
def test_lse_merge_random_partials(C, D):
    """Both merge forms (up to 16 chunks: one workgroup per row; more: one
    wave per 16 output dimensions), ragged chunk groups and dimensions,
    chunks and a whole row at lse = -inf, against the oracle merge."""
    import top_sparse_decode_amd as tsd
    rng = np.random.default_rng(3 + C + D)
    rows = 70
    o = rng.normal(size=(rows, C, D)).astype(np.float32)
    lse = (rng.normal(size=(rows, C)) * 5).astype(np.float32)
    lse[rng.random((rows, C)) < 0.3] = -np.inf
    lse[3] = -np.inf
    og = torch.from_numpy(o).to(DEV)
    lg = torch.from_numpy(lse).to(DEV)
    out = torch.empty((rows, D), device=DEV)
    out_lse = torch.empty(rows, device=DEV)
    tsd.lse_merge(og, lg, out, out_lse)
    torch.cuda.synchronize()
    check_merge(o, lse, out.cpu().numpy(), out_lse.cpu().numpy())
    assert (out[3] == 0).all() and torch.isneginf(out_lse[3])


def test_all_equal_scores_pick_lowest_indices():
    cfg = tsd_synth.config(QSA, B=2, lens=(3000, 200), top_k=256, chunks=4,
                           seed=120)
    wl = tsd_synth.make(cfg, DEV)
    wl["index_k"][:] = wl["index_k"][0]
    bufs = _run(wl)
    idx = bufs.idx.cpu().numpy()
    assert (idx[0] == np.arange(256)).all()
    assert (idx[1, :200] == np.arange(200)).all() and (idx[1, 200:] == -1).all()


def test_runs_are_bitwise_repeatable():
    cfg = tsd_synth.config(QSA, B=3, lens=(9000, 4097, 130), top_k=512,
                           chunks=8, seed=121)
    wl = tsd_synth.make(cfg, DEV)
    a = _run(wl)
    outs = [a.out.clone(), a.out_lse.clone(), a.idx.clone(), a.scores.clone()]
    b = _run(wl)
    for x, y in zip(outs, [b.out, b.out_lse, b.idx, b.scores]):
        assert torch.equal(torch.nan_to_num(x, nan=-1.0),
                           torch.nan_to_num(y, nan=-1.0))


def test_selection_covering_context_is_dense_attention():
    cfg = tsd_synth.config(QSA, B=2, lens=(1000, 77), top_k=1024, chunks=7,
                           seed=122)
    wl = tsd_synth.make(cfg, DEV)
    bufs = _run(wl)
    h = tsd_synth.to_host(wl)
    dense, dlse = oracle.dense_attention(h["q"], "bf16", h["k_pool"],
                                         h["v_pool"], "fp8_e4m3", h["k_scale"],
                                         h["v_scale"], h["page_table"],
                                         h["seq_lens"], h["num_pages"])
    assert np.abs(bufs.out.cpu().numpy() - dense).max() <= out_tol("fp8_e4m3")
    assert np.abs(bufs.out_lse.cpu().numpy() - dlse).max() <= out_tol("fp8_e4m3")


@pytest.mark.parametrize("fused,first", [(False, 6000), (True, 40000)],
                         ids=["separate-short", "fused-long"])
def test_graph_replay_matches_eager(fused, first):
    """The calls of a step captured in a HIP graph, replayed with fresh
    inputs copied in between (and eager work between replays), match the
    eager results of the same inputs on every replay: the separate calls on
    short rows (one-workgroup top-k), and sparse_index_topk on a row long
    enough for the chunked selection, whose histograms the in-scan pass
    fills and the resolve leaves zero for the next replay."""
    step = _step()
    cfg = tsd_synth.config(QSA, B=3, lens=(first, 4097, 130), top_k=512,
                           chunks=8, seed=130)
    wl = tsd_synth.make(cfg, DEV)
    bufs = step.StepBuffers(wl)
    plan = step.Plan(wl, bufs, fused=fused)
    plan.run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(torch.cuda.current_stream())
    gen = torch.Generator(device=DEV)
    gen.manual_seed(3)
    for rep in range(4):
        # mutate the query rows and the lengths in place, as a decode loop does
        wl["index_q"].copy_(tsd_synth.fp8_codes(
            torch.randn(wl["index_q"].shape, generator=gen, device=DEV)))
        wl["q"].copy_(torch.randn(wl["q"].shape, generator=gen,
                                  device=DEV).to(torch.bfloat16))
        wl["seq_lens"].copy_(torch.tensor([first - 7 * rep, 4097 - rep, 130 + rep],
                                          dtype=torch.int32, device=DEV))
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (bufs.idx, bufs.count, bufs.out, bufs.out_lse)]
        plan.run()
        torch.cuda.synchronize()
        for a, b in zip(got, (bufs.idx, bufs.count, bufs.out, bufs.out_lse)):
            assert torch.equal(a, b), f"replay {rep} differs from eager"
        assert not _hist_words(bufs.ws, bufs.rows).any(), "histograms left nonzero"


@pytest.mark.parametrize("name,over", [
    (QSA, dict(B=3, lens=(9000, 4097, 130), top_k=512, chunks=8)),
    (QSA, dict(B=2, lens=(700, 129), top_k=100, chunks=4, stale_tail=True)),
    (QSA, dict(B=2, lens=(2048, 50), top_k=2048, chunks=16)),
    # 32 rows of a 4,096-page table: 4,096 scan waves of 32 pages, more
    # than one pass of resident workgroups
    (QSA, dict(B=32, lens=(262144,) + tuple((i * 997) % 9000
                                             for i in range(1, 32)),
               top_k=256, chunks=4)),
    (DS8B, dict(B=2, lens=(3000, 700), top_k=200, chunks=3)),
    (DS7B, dict(B=2, H_q=8, H_kv=8, lens=(1500, 65), top_k=100, chunks=4,
                steps=0)),
    # rows past the one-workgroup top-k (label scan, digit-1 histogram,
    # filter, resolve), with one, two and three sub-blocks per page
    (DS8B, dict(B=3, lens=(40000, 27000, 300), top_k=1000, chunks=4)),
    (DS8B, dict(B=2, lens=(30000, 12345), r=64, n_outlier=40, top_k=500,
                chunks=4)),
    (DS8B, dict(B=1, H_q=48, H_kv=24, lens=(40000,), top_k=700, chunks=4)),
    # the general label kernel (r not a multiple of 8) on such rows
    (DS8B, dict(B=2, lens=(30000, 26000), r=24, n_outlier=24, top_k=500,
                chunks=4)),
])
def test_fused_score_select_matches_separate_calls(name, over):
    step = _step()
    wl = tsd_synth.make(tsd_synth.config(name, seed=140, **over), DEV)
    a = step.StepBuffers(wl)
    b = step.StepBuffers(wl)
    a.scores.fill_(float("nan"))
    b.scores.fill_(float("nan"))
    step.score(wl, a)
    step.select(wl, a)
    step.score_select(wl, b)
    torch.cuda.synchronize()
    for x, y in ((a.row_lens, b.row_lens), (a.idx, b.idx), (a.count, b.count)):
        assert torch.equal(x, y)
    assert torch.equal(torch.nan_to_num(a.scores, nan=-7.0),
                       torch.nan_to_num(b.scores, nan=-7.0))
    assert not _hist_words(b.ws, b.rows).any(), "histograms left nonzero"


@pytest.mark.gpu
@pytest.mark.parametrize("ranges", [
    ((0, 0, 8192),),                      # one whole scan workgroup's chunk
    ((0, 6000, 14000), (1, 40000, 41000)),  # across chunks, two rows
    ((0, 100000, 100040), (2, 29990, 30000)),  # a few tokens, a row's end
])
def test_fused_select_with_clustered_top_scores(ranges):
    """Long decode rows (4 x 4,096 pages, the index scan building the
    digit-1 histogram) whose top-k gathers in a few token ranges: the index
    keys there are set to six times the mean of their request's index
    heads. A chunk inside a long range keeps more survivors than its
    512-entry list holds and is re-read raw by the resolve; a short range
    puts a few of the top scores in one chunk. Scores, lengths and
    selections equal the separate calls bit for bit, and the selection
    equals the oracle's top-k of the GPU's own scores."""
    step = _step()
    wl = tsd_synth.make(tsd_synth.config(QSA, B=4, lens=(262144, 60000, 30000, 300),
                                         top_k=2048, chunks=4, seed=150), DEV)
    pt = wl["page_table"]
    iq = wl["index_q"].view(torch.float8_e4m3fn).float()  # [B, 16, 128]
    for b, lo, hi in ranges:
        t = torch.arange(lo, hi, device=DEV)
        slots = pt[b, t // 64].long() * 64 + t % 64
        boost = (6.0 * iq[b].mean(dim=0)).clamp(-448, 448)
        wl["index_k"][slots] = tsd_synth.fp8_codes(boost.expand(len(t), -1).contiguous())
    a = step.StepBuffers(wl)
    b_ = step.StepBuffers(wl)
    a.scores.fill_(float("nan"))
    b_.scores.fill_(float("nan"))
    step.score(wl, a)
    step.select(wl, a)
    step.score_select(wl, b_)
    torch.cuda.synchronize()
    for x, y in ((a.row_lens, b_.row_lens), (a.idx, b_.idx), (a.count, b_.count)):
        assert torch.equal(x, y)
    assert torch.equal(torch.nan_to_num(a.scores, nan=-7.0),
                       torch.nan_to_num(b_.scores, nan=-7.0))
    assert not _hist_words(b_.ws, b_.rows).any(), "histograms left nonzero"
    S = np.nan_to_num(b_.scores.cpu().numpy(), nan=0.0)
    ridx, rcnt = oracle.topk(S, b_.row_lens.cpu().numpy(), 2048)
    assert np.array_equal(b_.idx.cpu().numpy(), ridx)
    assert np.array_equal(b_.count.cpu().numpy(), rcnt)
    # the boosted range holds the top of row 0 (the case is what it says)
    lo0, hi0 = ranges[0][1], ranges[0][2]
    sel0 = b_.idx[0].cpu().numpy()
    assert ((sel0 >= lo0) & (sel0 < hi0)).sum() >= 0.9 * min(2048, hi0 - lo0)


def _prefill_case(lens, R, seed, stale_tail=False):
    cfg = tsd_synth.config(QSA, B=len(lens), lens=lens, top_k=200, chunks=4,
                           seed=seed, stale_tail=stale_tail)
    wl = tsd_synth.make(cfg, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    B = len(lens)
    wl["index_q"] = tsd_synth.fp8_codes(
        torch.randn((B * R, 16, 128), generator=g, device=DEV))
    wl["index_w"] = torch.rand((B * R, 16), generator=g, device=DEV)
    # positions spread over each request, including 0 and the last token
    qp = []
    for b, n in enumerate(lens):
        p = torch.linspace(0, max(n - 1, 0), R).round().to(torch.int32)
        qp.append(p)
    wl["q_pos"] = torch.cat(qp).to(DEV)
    wl["rows_per_req"] = R
    return wl


@pytest.mark.parametrize("lens,R", [((20000,), 130), ((5000, 70000), 64),
                                    ((16384 + 77, 300), 65)])
def test_prefill_kernel_and_decode_scan_against_oracle(lens, R):
    """Rows of a request >= 64 take the tiled prefill kernel (FP8 MFMA); the
    same rows scored one at a time take the decode scan (bf16 MFMA on the
    widened codes, FP32 accumulation). Both match the oracle: the decode
    scan within half the tie window of every row (its error is FP32
    rounding), the prefill kernel within the FP8 score tolerance; the row
    lengths agree."""
    import top_sparse_decode_amd as tsd
    from gpu_checks import score_error_vs_window
    wl = _prefill_case(lens, R, seed=150)
    B = len(lens)
    stride = wl["page_table"].shape[1] * 64
    tiled = torch.full((B * R, stride), float("nan"), device=DEV)
    rl = torch.empty(B * R, dtype=torch.int32, device=DEV)
    tsd.sparse_index_score("qsa", tiled, wl["page_table"], wl["seq_lens"],
                           wl["num_pages"], index_q=wl["index_q"],
                           index_w=wl["index_w"], index_k_pool=wl["index_k"],
                           q_pos=wl["q_pos"], rows_per_req=R, row_lens_out=rl)
    single = torch.full_like(tiled, float("nan"))
    for b in range(B):
        for r in range(R):
            i = b * R + r
            tsd.sparse_index_score(
                "qsa", single[i:i + 1], wl["page_table"][b:b + 1],
                wl["seq_lens"][b:b + 1], wl["num_pages"],
                index_q=wl["index_q"][i:i + 1], index_w=wl["index_w"][i:i + 1],
                index_k_pool=wl["index_k"], q_pos=wl["q_pos"][i:i + 1])
    torch.cuda.synchronize()
    expect = torch.minimum(wl["q_pos"].long() + 1,
                           wl["seq_lens"].long().repeat_interleave(R))
    assert torch.equal(rl.long(), expect)
    h = tsd_synth.to_host(wl)
    rows = np.arange(0, B * R, max(1, (B * R) // 24))
    sub = dict(h)
    sub["index_q"], sub["index_w"] = h["index_q"][rows], h["index_w"][rows]
    sub["q_pos"] = h["q_pos"][rows]
    ref = np.concatenate([oracle.qsa_scores(
        h["index_q"][i:i + 1], h["index_w"][i:i + 1], h["index_k"],
        h["page_table"][i // R:i // R + 1], h["seq_lens"][i // R:i // R + 1],
        h["num_pages"], q_pos=h["q_pos"][i:i + 1],
        score_stride=stride) for i in rows])
    n_rows = expect.cpu().numpy()[rows]
    check_scores(tiled.cpu().numpy()[rows], ref, n_rows, score_tol("qsa"))
    check_scores(single.cpu().numpy()[rows], ref, n_rows, score_tol("qsa"))
    ratio = score_error_vs_window(single.cpu().numpy()[rows], ref, n_rows, 200)
    assert 2 * ratio.max() <= 1.0, ratio


def test_prefill_kernel_against_oracle():
    wl = _prefill_case((3000, 1300), 70, seed=151, stale_tail=True)
    step = _step()
    bufs = step.StepBuffers(wl)
    bufs.scores.fill_(float("nan"))
    step.score_select(wl, bufs)
    torch.cuda.synchronize()
    h = tsd_synth.to_host(wl)
    rl = oracle_row_lens(h)
    np.testing.assert_array_equal(bufs.row_lens.cpu().numpy(), rl)
    gs = bufs.scores.cpu().numpy()
    check_scores(gs, oracle_scores(h), rl, score_tol("qsa"))
    check_topk_identical(gs, rl, 200, bufs.idx.cpu().numpy(),
                         bufs.count.cpu().numpy())
