"""GPU parity at the workloads' full sizes, through the launch path the
benchmark times: ``step.Plan`` issuing either sparse_index_score +
topk_select or the fused sparse_index_topk (which picks the in-scan
histogram variants of the index scan at these shapes), both checked. The
oracle checks whole rows it can finish in seconds (scores, identical top-k
on the GPU's scores, end-to-end selection within the tie window, attention
on the GPU's selection) and sampled score points on every other row; the
merge is checked on every row."""
import numpy as np
import pytest
import torch

import oracle
import tsd_synth
from gpu_checks import (check_attention_on, check_merge, check_scores,
                        check_sets_within_window, check_topk_identical,
                        oracle_row_lens, out_tol, score_error_vs_window,
                        score_tol)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import top_sparse_decode_amd  # noqa: F401


def _step():
    import top_sparse_decode_amd.step as step
    return step


def _oracle_rows(h, rows):
    """Oracle f64 scores of the listed rows only, [len(rows), stride]."""
    rows = list(rows)
    if h["mode"] == "ds":
        H_kv = h["channel_idx"].shape[0]
        out = []
        for r in rows:
            b, g = divmod(r, H_kv)
            s = oracle.ds_scores(h["q"][b:b + 1], h["q_enc"],
                                 h["channel_idx"], h["label_pool"],
                                 h["kv_enc"], h["page_table"][b:b + 1],
                                 h["seq_lens"][b:b + 1], h["num_pages"])
            out.append(s[g])
        return np.stack(out)
    R = h.get("rows_per_req", 1)
    out = []
    for r in rows:
        b = r // R
        qp = None if h.get("q_pos") is None else h["q_pos"][r:r + 1]
        s = oracle.qsa_scores(h["index_q"][r:r + 1], h["index_w"][r:r + 1],
                              h["index_k"], h["page_table"][b:b + 1],
                              h["seq_lens"][b:b + 1], h["num_pages"],
                              rows_per_req=1, q_pos=qp)
        out.append(s[0])
    return np.stack(out)


def _sampled_points(h, gs, rl, tol, per_row=64, seed=0):
    rng = np.random.default_rng(seed)
    rows, ts = [], []
    for r in range(gs.shape[0]):
        n = int(rl[r])
        if n == 0:
            continue
        t = rng.integers(0, n, size=per_row)
        t[0], t[-1] = 0, n - 1
        rows.extend([r] * per_row)
        ts.extend(t.tolist())
    rows, ts = np.array(rows), np.array(ts)
    if h["mode"] == "ds":
        ref = oracle.ds_score_points(h["q"], h["q_enc"], h["channel_idx"],
                                     h["label_pool"], h["kv_enc"],
                                     h["page_table"], h["seq_lens"],
                                     h["num_pages"], rows, ts)
    else:
        ref = oracle.qsa_score_points(h["index_q"], h["index_w"], h["index_k"],
                                      h["page_table"], h["seq_lens"],
                                      h["num_pages"], rows, ts,
                                      rows_per_req=h.get("rows_per_req", 1),
                                      q_pos=h.get("q_pos"))
    err = np.abs(gs[rows, ts].astype(np.float64) - ref).max()
    assert err <= tol, err


def _check_layer(wl, bufs, full_rows, check_batches=None, label=""):
    h = tsd_synth.to_host(wl)
    B, k, C = wl["B"], wl["top_k"], wl["chunks"]
    rl = oracle_row_lens(h)
    np.testing.assert_array_equal(bufs.row_lens.cpu().numpy(), rl)
    gs = bufs.scores.cpu().numpy()
    gidx, gcnt = bufs.idx.cpu().numpy(), bufs.count.cpu().numpy()
    tol = score_tol(wl["mode"])
    _sampled_points(h, gs, rl, tol)
    # whole rows
    ref64 = _oracle_rows(h, full_rows)
    worst = check_scores(gs[full_rows], ref64, rl[full_rows], tol)
    ratio = score_error_vs_window(gs[full_rows], ref64, rl[full_rows], k)
    print(f"scores {label}: max |gpu - oracle| over whole rows {worst:.3g}, "
          f"max error / tie window {ratio.max():.3g}", flush=True)
    if wl["mode"] == "qsa":
        # the decode scan's FP32 accumulation keeps every score within half
        # the tie window, so the end-to-end sets hold for any data
        assert 2 * ratio.max() <= 1.0, ratio
    check_topk_identical(gs, rl, k, gidx, gcnt, rows=full_rows)
    ref32 = ref64.astype(np.float32)
    ridx, rcnt = oracle.topk(ref32, rl[full_rows], k)
    check_sets_within_window(gidx[full_rows], gcnt[full_rows], ridx, rcnt,
                             ref32, rl[full_rows], k, rows=full_rows,
                             label=label)
    op, lp = bufs.o_part.cpu().numpy(), bufs.lse_part.cpu().numpy()
    if check_batches is None:
        check_batches = range(B)
    check_attention_on(h, gidx.reshape(B, bufs.H_sel, k),
                       gcnt.reshape(B, bufs.H_sel), C, op, lp,
                       out_tol(wl["kv_enc"]), batch=list(check_batches))
    check_merge(op, lp, bufs.out.cpu().numpy(), bufs.out_lse.cpu().numpy())


FUSED = pytest.mark.parametrize("fused", [False, True],
                                ids=["separate", "fused"])


def _run(wl, fused):
    """One step through step.Plan, as bench.py launches it."""
    step = _step()
    bufs = step.StepBuffers(wl)
    bufs.scores.fill_(float("nan"))
    step.Plan(wl, bufs, fused=fused).run()
    torch.cuda.synchronize()
    return bufs


@FUSED
def test_full_ds_tiny_b1_l4096(fused):
    wl = tsd_synth.make("ds_tiny_b1_l4096", DEV)
    bufs = _run(wl, fused)
    _check_layer(wl, bufs, full_rows=[0], label=f"ds_tiny fused={fused}")


@FUSED
def test_full_ds_llama31_8b_b3_l60000(fused):
    wl = tsd_synth.make("ds_llama31_8b_b3_l60000", DEV)
    bufs = _run(wl, fused)
    _check_layer(wl, bufs, full_rows=list(range(24)),
                 label=f"ds_llama31_8b fused={fused}")


@FUSED
def test_full_ds_llama7b_b3_l20000_200_steps(fused):
    """200 decode steps, each appending one token per request: lengths run
    20,001 .. 20,200 with a fresh query per step, written in place so that
    one Plan (marshalled once, as in bench.py) serves every step; steps 0,
    1, 99 and 199 are checked against the oracle."""
    step = _step()
    wl = tsd_synth.make("ds_llama7b_b3_l20000_s200", DEV)
    bufs = step.StepBuffers(wl)
    plan = step.Plan(wl, bufs, fused=fused)
    base = wl["seq_lens"].clone()
    checked = {0, 1, 99, 199}
    for s in range(200):
        wl["seq_lens"].copy_(base + s)
        wl["q"].copy_(wl["step_q"][s])
        if s in checked:
            bufs.scores.fill_(float("nan"))
        plan.run()
        if s in checked:
            torch.cuda.synchronize()
            print(f"step {s} len {int(wl['seq_lens'][0])}", flush=True)
            _check_layer(wl, bufs, full_rows=[0, 31, 32, 95],
                         label=f"ds_llama7b step {s} fused={fused}")
    torch.cuda.synchronize()


def test_full_ds_llama7b_b3_200_steps_appended_on_gpu():
    """The 200-step workload with each step's new token stored by kv_append
    (K, V and its label row) before the step, from rows held aside; the
    slots start as garbage. The step is the fused plan bench.py times.
    Steps 0, 100 and 199 are checked against the oracle and the pools end
    equal to the generated ones."""
    import top_sparse_decode_amd as tsd
    step = _step()
    wl = tsd_synth.make("ds_llama7b_b3_l20000_s200", DEV)
    bufs = step.StepBuffers(wl)
    plan = step.Plan(wl, bufs, fused=True)
    base = wl["seq_lens"].clone()
    pt = wl["page_table"]
    B = base.shape[0]
    pos = (base.long() - 1)[:, None] + torch.arange(200, device=DEV)[None]
    slots = (pt.long().gather(1, pos // 64) * 64 + pos % 64)  # [B, 200]
    keep = {n: wl[n].clone() for n in ("k_pool", "v_pool", "label_pool")}
    k_rows = wl["k_pool"][slots]                              # [B, 200, H, D]
    v_rows = wl["v_pool"][slots]
    for n in keep:
        wl[n][slots] = torch.randn_like(wl[n][slots])
    one = torch.ones(B, dtype=torch.int32, device=DEV)
    for s in range(200):
        tsd.kv_append(pt, wl["num_pages"], pos[:, s].to(torch.int32), one, 1,
                      k_new=k_rows[:, s:s + 1].contiguous(),
                      v_new=v_rows[:, s:s + 1].contiguous(),
                      k_pool=wl["k_pool"], v_pool=wl["v_pool"],
                      channel_idx=wl["channel_idx"],
                      label_pool=wl["label_pool"])
        wl["seq_lens"].copy_(base + s)
        wl["q"].copy_(wl["step_q"][s])
        if s in (0, 100, 199):
            bufs.scores.fill_(float("nan"))
        plan.run()
        if s in (0, 100, 199):
            torch.cuda.synchronize()
            print(f"step {s} len {int(wl['seq_lens'][0])}", flush=True)
            _check_layer(wl, bufs, full_rows=[0, 95],
                         label=f"ds_llama7b appended step {s}")
    torch.cuda.synchronize()
    for n, t in keep.items():
        assert torch.equal(wl[n], t), n


@FUSED
def test_full_qsa_decode_b8_l262144(fused):
    """The benchmark's workload: every request's row checked whole."""
    wl = tsd_synth.make("qsa_decode_b8_l262144_k2048", DEV)
    bufs = _run(wl, fused)
    _check_layer(wl, bufs, full_rows=list(range(8)),
                 label=f"qsa_b8_l262144 fused={fused}")


@FUSED
def test_full_qsa_two_requests_eight_pages_per_scan_wave(fused):
    """Two requests on a 4,096-page table (8,192 pages): the scan takes 8
    pages per wave, the form the 8 x 262,144 (32) and 1 x 1,048,576 (16)
    workloads and the small cases (4) leave out."""
    wl = tsd_synth.make(tsd_synth.config("qsa_decode_b8_l262144_k2048", B=2,
                                         lens=(262144, 150001), seed=161), DEV)
    bufs = _run(wl, fused)
    _check_layer(wl, bufs, full_rows=[1],
                 label=f"qsa b2 {'fused' if fused else 'separate'}")


@FUSED
def test_full_qsa_decode_b1_l1048576(fused):
    wl = tsd_synth.make("qsa_decode_b1_l1048576_k2048", DEV)
    bufs = _run(wl, fused)
    _check_layer(wl, bufs, full_rows=[0], label=f"qsa_b1_l1048576 fused={fused}")


@pytest.mark.parametrize("name", ["qsa_decode_b8_l262144_k2048",
                                  "qsa_decode_b1_l1048576_k2048",
                                  "ds_llama31_8b_b3_l60000"])
def test_full_fused_equals_separate(name):
    """The fused plan (in-scan digit-1 histogram at these shapes) and the
    separate calls give bit-identical scores, lengths, selections and
    outputs at the timed shapes."""
    wl = tsd_synth.make(name, DEV)
    a = _run(wl, fused=False)
    b = _run(wl, fused=True)
    for x, y in ((a.row_lens, b.row_lens), (a.idx, b.idx), (a.count, b.count),
                 (a.o_part, b.o_part), (a.lse_part, b.lse_part),
                 (a.out, b.out), (a.out_lse, b.out_lse)):
        assert torch.equal(x, y)
    assert torch.equal(torch.nan_to_num(a.scores, nan=-7.0),
                       torch.nan_to_num(b.scores, nan=-7.0))


def test_full_sharded_select_b1_l1048576_w4():
    """The 1M-token request split over 4 page-owner shards of 262,144 tokens
    (each one GPU's share): per-shard score and top-k, then the exact merge,
    equals the unsharded selection bit for bit."""
    from gpu_checks import sharded_qsa_select
    wl = tsd_synth.make("qsa_decode_b1_l1048576_k2048", DEV)
    bufs = _run(wl, fused=True)
    idx, cnt, _, lens = sharded_qsa_select(wl, 4, 2048)
    torch.cuda.synchronize()
    assert lens[:, 0].tolist() == [262144] * 4
    assert torch.equal(idx, bufs.idx.view(1, 2048))
    assert torch.equal(cnt, bufs.count.view(1))


def test_full_qsa_prefill_r2048_l1048576():
    """Chunked-prefill indexer pass: 2,048 causal query rows against all
    1,048,576 index keys, then per-row top-k, through the separate calls and
    through the fused sparse_index_topk (identical results). Rows 0, 1023
    and 2047 are checked whole against the oracle (scores and the
    end-to-end selection within the tie window); the top-k of 8 rows is
    compared with the oracle's top-k of the same scores; every row's scores
    are sampled at its first and last key and two random keys."""
    step = _step()
    wl = tsd_synth.make("qsa_prefill_r2048_l1048576_k2048", DEV)
    bufs = step.StepBuffers(wl)
    bufs.scores.fill_(float("nan"))
    step.score(wl, bufs)
    step.select(wl, bufs)
    torch.cuda.synchronize()
    h = tsd_synth.to_host(wl)
    rl = oracle_row_lens(h)
    np.testing.assert_array_equal(bufs.row_lens.cpu().numpy(), rl)
    rows = [0, 1023, 2047]
    gs_rows = bufs.scores[rows].cpu().numpy()
    ref64 = _oracle_rows(h, rows)
    worst = check_scores(gs_rows, ref64, rl[rows], score_tol("qsa"))
    ratio = score_error_vs_window(gs_rows, ref64, rl[rows], 2048)
    print(f"scores prefill: max |gpu - oracle| over rows {rows} {worst:.3g}, "
          f"max error / tie window {ratio.max():.3g}", flush=True)
    gidx, gcnt = bufs.idx.cpu().numpy(), bufs.count.cpu().numpy()
    ref32 = ref64.astype(np.float32)
    ridx, rcnt = oracle.topk(ref32, rl[rows], 2048)
    check_sets_within_window(gidx[rows], gcnt[rows], ridx, rcnt, ref32,
                             rl[rows], 2048, rows=rows, label="prefill")
    sel_rows = [0, 1, 511, 1023, 1024, 1535, 2046, 2047]
    ridx, rcnt = oracle.topk(bufs.scores[sel_rows].cpu().numpy(),
                             rl[sel_rows], 2048)
    np.testing.assert_array_equal(gidx[sel_rows], ridx)
    np.testing.assert_array_equal(gcnt[sel_rows], rcnt)
    # 4 sampled points on every row: its first and last key, 2 random keys
    rng = np.random.default_rng(1)
    sample_rows = np.repeat(np.arange(2048), 4)
    ts = np.array([[0, rl[r] - 1, rng.integers(0, rl[r]), rng.integers(0, rl[r])]
                   for r in range(2048)]).reshape(-1)
    got = bufs.scores[torch.from_numpy(sample_rows).to(DEV),
                      torch.from_numpy(ts).to(DEV)].cpu().numpy()
    ref = oracle.qsa_score_points(h["index_q"], h["index_w"], h["index_k"],
                                  h["page_table"], h["seq_lens"],
                                  h["num_pages"], sample_rows, ts,
                                  rows_per_req=2048, q_pos=h["q_pos"])
    assert np.abs(got - ref).max() <= score_tol("qsa")
    # the fused call: identical scores, lengths and selections
    idx_sep, cnt_sep = bufs.idx.clone(), bufs.count.clone()
    sc_sep = bufs.scores
    fused = step.StepBuffers(wl)
    fused.scores.fill_(float("nan"))
    step.score_select(wl, fused)
    torch.cuda.synchronize()
    assert torch.equal(fused.idx, idx_sep)
    assert torch.equal(fused.count, cnt_sep)
    assert torch.equal(fused.row_lens, bufs.row_lens)
    assert torch.equal(torch.nan_to_num(fused.scores, nan=-7.0),
                       torch.nan_to_num(sc_sep, nan=-7.0))
