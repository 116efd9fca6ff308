"""CPU oracle for top-k sparse decode attention: a thin ctypes wrapper over
``tsd_oracle.c`` (plain C11, double-precision accumulation).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package. The product library
(``top_sparse_decode_amd``) never imports, links or calls it, and the two share
no code: the oracle decodes every stored format from its definition and
computes each step exactly as the pages define it (see ``tsd_oracle.c`` for
the page and section each function follows).

Arrays are numpy, C-contiguous, in the library's layouts. Half-precision and
FP8 tensors are passed as their raw codes (``uint16`` / ``uint8``) together
with an encoding tag (``"bf16"``, ``"fp16"``, ``"fp8_e4m3"``, ``"f32"``).
Results are float64 except top-k indices.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "tsd_oracle.c")
# TSD_ORACLE_LIB names another build of the same source (the tests'
# sanitizer build), used as it is.
LIB_PATH = os.environ.get("TSD_ORACLE_LIB") or os.path.join(_DIR, "libtsd_oracle.so")

DTYPE = {"bf16": 1, "fp16": 2, "fp8_e4m3": 3, "f32": 4}
_ERR = {-1: "bad argument", -2: "page id out of range",
        -3: "token index out of range", -4: "NaN score"}


class OracleError(RuntimeError):
    pass


def build(out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (no HIP headers, no GPU code)."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
           _SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.environ.get("TSD_ORACLE_LIB") and (
            not os.path.exists(LIB_PATH)
            or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    sig = {
        "tsd_oracle_decode_fp8e4m3": (D, [ctypes.c_uint8]),
        "tsd_oracle_decode_bf16": (D, [ctypes.c_uint16]),
        "tsd_oracle_decode_fp16": (D, [ctypes.c_uint16]),
        "tsd_oracle_slot": (L, [P, L, I, L, I, L]),
        "tsd_oracle_ds_scores": (I, [I, I, I, I, I, P, I, P, P, I, P, L, P, L,
                                     I, P, L]),
        "tsd_oracle_ds_score_points": (I, [I, I, I, I, I, P, I, P, P, I, P, L,
                                           P, L, I, L, P, P, P]),
        "tsd_oracle_qsa_scores": (I, [I, I, I, I, P, P, P, P, L, P, P, L, I,
                                      P, L]),
        "tsd_oracle_qsa_score_points": (I, [I, I, I, I, P, P, P, P, L, P, P,
                                            L, I, L, P, P, P]),
        "tsd_oracle_topk": (I, [P, L, I, P, I, P, P]),
        "tsd_oracle_topk_merge_sharded": (I, [P, L, P, P, I, I, I, I, I, P,
                                              P]),
        "tsd_oracle_encode_fp8e4m3": (ctypes.c_uint8, [D]),
        "tsd_oracle_index_k_compress": (I, [I, I, P, P, L, L, P, P, P, L, L,
                                            I, I, P]),
        "tsd_oracle_expand_blocks": (I, [I, P, P, I, I, P, I, P, P]),
        "tsd_oracle_kv_append": (I, [I, L, P, L, I, P, P, I, I, I, P, P, I, P,
                                     P, I, P, P, P, I, P, P, I, P, I]),
        "tsd_oracle_sparse_attention": (I, [I, I, I, I, I, I, I, P, I, P, P, I,
                                            P, P, P, L, P, L, I, P, P, D, P,
                                            P]),
        "tsd_oracle_lse_merge": (I, [P, P, I, I, I, P, P]),
        "tsd_oracle_dense_attention": (I, [I, I, I, I, P, I, P, P, I, P, P, P,
                                           L, P, L, I, D, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc):
    if rc != 0:
        raise OracleError(_ERR.get(rc, f"oracle error {rc}"))


def _codes(a, enc):
    """Raw codes of a stored tensor for the given encoding."""
    if enc == "fp8_e4m3":
        return _c(a, np.uint8)
    if enc in ("bf16", "fp16"):
        return _c(a, np.uint16)
    if enc == "f32":
        return _c(a, np.float32)
    raise ValueError(enc)


# ------------------------------------------------------------------ decoders
def decode_fp8_e4m3(code: int) -> float:
    return _load().tsd_oracle_decode_fp8e4m3(int(code))


def encode_fp8_e4m3(x: float) -> int:
    """Nearest OCP E4M3 code (ties to even, saturating at 448)."""
    return int(_load().tsd_oracle_encode_fp8e4m3(float(x)))


def decode_bf16(bits: int) -> float:
    return _load().tsd_oracle_decode_bf16(int(bits))


def decode_fp16(bits: int) -> float:
    return _load().tsd_oracle_decode_fp16(int(bits))


def slot(page_table, b, t, page_size, num_pages) -> int:
    pt = _c(page_table, np.int32)
    return _load().tsd_oracle_slot(_ptr(pt), pt.shape[1], b, t, page_size,
                                   num_pages)


# ------------------------------------------------------------------- scores
def ds_scores(q, q_enc, chan, label, label_enc, page_table, seq_lens,
              num_pages, page_size=64, score_stride=None):
    """Double-sparsity label scores, float64 [B*H_kv, score_stride]; entries
    at t >= len are NaN (never written)."""
    B, H_q, D = q.shape
    H_kv, r = chan.shape
    qc, lc = _codes(q, q_enc), _codes(label, label_enc)
    ch, pt, sl = _c(chan, np.int32), _c(page_table, np.int32), _c(seq_lens, np.int32)
    stride = score_stride or max(1, int(sl.max()) if sl.size else 1)
    out = np.full((B * H_kv, stride), np.nan)
    _check(_load().tsd_oracle_ds_scores(
        B, H_q, H_kv, D, r, _ptr(qc), DTYPE[q_enc], _ptr(ch), _ptr(lc),
        DTYPE[label_enc], _ptr(pt), pt.shape[1], _ptr(sl), num_pages,
        page_size, _ptr(out), stride))
    return out


def ds_score_points(q, q_enc, chan, label, label_enc, page_table, seq_lens,
                    num_pages, rows, ts, page_size=64):
    B, H_q, D = q.shape
    H_kv, r = chan.shape
    qc, lc = _codes(q, q_enc), _codes(label, label_enc)
    ch, pt, sl = _c(chan, np.int32), _c(page_table, np.int32), _c(seq_lens, np.int32)
    pr, pt_t = _c(rows, np.int32), _c(ts, np.int64)
    out = np.empty(pr.shape[0])
    _check(_load().tsd_oracle_ds_score_points(
        B, H_q, H_kv, D, r, _ptr(qc), DTYPE[q_enc], _ptr(ch), _ptr(lc),
        DTYPE[label_enc], _ptr(pt), pt.shape[1], _ptr(sl), num_pages,
        page_size, pr.shape[0], _ptr(pr), _ptr(pt_t), _ptr(out)))
    return out


def qsa_scores(index_q, index_w, index_k, page_table, seq_lens, num_pages,
               rows_per_req=1, q_pos=None, page_size=64, score_stride=None):
    """QSA index scores, float64 [rows, score_stride] (NaN beyond each row's
    key count)."""
    rows, H_i, D_i = index_q.shape
    iq, iw, ik = _c(index_q, np.uint8), _c(index_w, np.float32), _c(index_k, np.uint8)
    pt, sl = _c(page_table, np.int32), _c(seq_lens, np.int32)
    qp = None if q_pos is None else _c(q_pos, np.int32)
    stride = score_stride or max(1, int(sl.max()) if sl.size else 1)
    out = np.full((rows, stride), np.nan)
    _check(_load().tsd_oracle_qsa_scores(
        rows, rows_per_req, H_i, D_i, _ptr(iq), _ptr(iw), _ptr(ik), _ptr(pt),
        pt.shape[1], _ptr(sl), _ptr(qp), num_pages, page_size, _ptr(out),
        stride))
    return out


def qsa_score_points(index_q, index_w, index_k, page_table, seq_lens,
                     num_pages, rows, ts, rows_per_req=1, q_pos=None,
                     page_size=64):
    nrows, H_i, D_i = index_q.shape
    iq, iw, ik = _c(index_q, np.uint8), _c(index_w, np.float32), _c(index_k, np.uint8)
    pt, sl = _c(page_table, np.int32), _c(seq_lens, np.int32)
    qp = None if q_pos is None else _c(q_pos, np.int32)
    pr, pt_t = _c(rows, np.int32), _c(ts, np.int64)
    out = np.empty(pr.shape[0])
    _check(_load().tsd_oracle_qsa_score_points(
        nrows, rows_per_req, H_i, D_i, _ptr(iq), _ptr(iw), _ptr(ik), _ptr(pt),
        pt.shape[1], _ptr(sl), _ptr(qp), num_pages, page_size, pr.shape[0],
        _ptr(pr), _ptr(pt_t), _ptr(out)))
    return out


# -------------------------------------------------------------------- top-k
def topk(scores, row_lens, k):
    """Exact top-k on float32 scores [rows, stride] -> (idx int32 [rows, k],
    count int32 [rows])."""
    s = _c(scores, np.float32)
    if s.ndim == 1:
        s = s[None, :]
    rows, stride = s.shape
    rl = _c(row_lens, np.int32)
    idx = np.empty((rows, k), np.int32)
    cnt = np.empty(rows, np.int32)
    _check(_load().tsd_oracle_topk(_ptr(s), stride, rows, _ptr(rl), k,
                                   _ptr(idx), _ptr(cnt)))
    return idx, cnt


def kv_append(page_table, num_pages, positions, n_new, max_new, *,
              k_new=None, v_new=None, new_enc="bf16", k_pool=None,
              v_pool=None, kv_enc="bf16", k_scale=None, v_scale=None,
              channel_idx=None, label_pool=None, index_k_new=None,
              index_enc="bf16", index_k_pool=None, page_size=64):
    """Cache append on host copies: returns the updated pools as a dict
    (k_pool, v_pool, k_scale, v_scale, label_pool, index_k_pool; absent
    ones None). New rows are raw codes of their encodings: k_new/v_new
    [B, max_new, H_kv, D] 16-bit, index_k_new [B, max_new, 128]."""
    pt = _c(page_table, np.int32)
    B, pt_stride = pt.shape
    pos = _c(positions, np.int32)
    nn = _c(n_new, np.int32)
    out = {}
    H_kv = D = r = 0
    kn = vn = kp = vp = ks = vs = None
    if k_pool is not None:
        kn, vn = _codes(k_new, new_enc).copy(), _codes(v_new, new_enc).copy()
        H_kv, D = kn.shape[2], kn.shape[3]
        kp, vp = _codes(k_pool, kv_enc).copy(), _codes(v_pool, kv_enc).copy()
        if kv_enc == "fp8_e4m3":
            ks, vs = _c(k_scale, np.float32).copy(), _c(v_scale, np.float32).copy()
    ci = lp = None
    if label_pool is not None:
        kn = _codes(k_new, new_enc).copy() if kn is None else kn
        H_kv, D = kn.shape[2], kn.shape[3]
        ci = _c(channel_idx, np.int32)
        r = ci.shape[1]
        lp = _codes(label_pool, new_enc).copy()
    ikn = ikp = None
    D_i = 0
    if index_k_pool is not None:
        ikn = _codes(index_k_new, index_enc).copy()
        D_i = ikn.shape[2]
        ikp = _c(index_k_pool, np.uint8).copy()
    _check(_load().tsd_oracle_kv_append(
        B, pt_stride, _ptr(pt), int(num_pages), page_size, _ptr(pos),
        _ptr(nn), int(max_new), H_kv, D, _ptr(kn), _ptr(vn), DTYPE[new_enc],
        _ptr(kp), _ptr(vp), DTYPE[kv_enc], _ptr(ks), _ptr(vs), _ptr(ci), r,
        _ptr(lp), _ptr(ikn), DTYPE[index_enc], _ptr(ikp), D_i))
    out.update(k_pool=kp, v_pool=vp, k_scale=ks, v_scale=vs, label_pool=lp,
               index_k_pool=ikp)
    return out


def index_k_compress(index_k, page_table, num_pages, seq_lens, from_block,
                     cpage_table, num_cpages, ck_pool, Bs, page_size=64):
    """Block-compressed index keys on host copies -> updated ck_pool
    (uint8 [cslots, D_i])."""
    ik = _c(index_k, np.uint8)
    pt = _c(page_table, np.int32)
    cpt = _c(cpage_table, np.int32)
    out = _c(ck_pool, np.uint8).copy()
    B = pt.shape[0]
    _check(_load().tsd_oracle_index_k_compress(
        B, Bs, _ptr(ik), _ptr(pt), pt.shape[1], int(num_pages),
        _ptr(_c(seq_lens, np.int32)), _ptr(_c(from_block, np.int32)),
        _ptr(cpt), cpt.shape[1], int(num_cpages), page_size, ik.shape[1],
        _ptr(out)))
    return out


def expand_blocks(sel, count, Bs, row_lens, kt):
    """Selected blocks [rows, kb] -> (tokens int32 [rows, kt], count)."""
    sl = _c(sel, np.int32)
    rows, kb = sl.shape
    tok = np.empty((rows, kt), np.int32)
    cnt = np.empty(rows, np.int32)
    _check(_load().tsd_oracle_expand_blocks(
        rows, _ptr(sl), _ptr(_c(count, np.int32)), kb, Bs,
        _ptr(_c(row_lens, np.int32)), kt, _ptr(tok), _ptr(cnt)))
    return tok, cnt


def topk_merge_sharded(scores, idx, count, k, page_size=64):
    """Exact global top-k from W page-owner shards: scores f32 [W, rows,
    stride] (shard-local order), idx int32 [W, rows, kl] (local top-k lists),
    count int32 [W, rows] -> (global idx int32 [rows, k], count [rows])."""
    s = _c(scores, np.float32)
    ix = _c(idx, np.int32)
    ct = _c(count, np.int32)
    W, rows, stride = s.shape
    kl = ix.shape[2]
    assert ix.shape[:2] == (W, rows) and ct.shape == (W, rows)
    out = np.empty((rows, k), np.int32)
    cnt = np.empty(rows, np.int32)
    _check(_load().tsd_oracle_topk_merge_sharded(
        _ptr(s), stride, _ptr(ix), _ptr(ct), W, rows, kl, page_size, k,
        _ptr(out), _ptr(cnt)))
    return out, cnt


def shard_row_order(n, W, page_size=64):
    """Global tokens of each shard in local order, for a row of n tokens
    whose logical pages are owned by p % W: a list of W int64 arrays."""
    t = np.arange(n, dtype=np.int64)
    owner = (t // page_size) % W
    return [t[owner == w] for w in range(W)]


# ---------------------------------------------------------------- attention
def sparse_attention(q, q_enc, k_pool, v_pool, kv_enc, k_scale, v_scale,
                     page_table, seq_lens, num_pages, idx, count, chunks,
                     softmax_scale=None, page_size=64):
    """Chunked sparse GQA attention -> (o_part [B,H_q,C,D], lse_part
    [B,H_q,C]) float64."""
    B, H_q, D = q.shape
    H_kv = k_pool.shape[1]
    H_sel, k = idx.shape[1], idx.shape[2]
    qc = _codes(q, q_enc)
    kc, vc = _codes(k_pool, kv_enc), _codes(v_pool, kv_enc)
    ks = None if k_scale is None else _c(k_scale, np.float32)
    vs = None if v_scale is None else _c(v_scale, np.float32)
    pt, sl = _c(page_table, np.int32), _c(seq_lens, np.int32)
    ix, ct = _c(idx, np.int32), _c(count, np.int32)
    scale = softmax_scale if softmax_scale is not None else 1.0 / np.sqrt(D)
    o = np.empty((B, H_q, chunks, D))
    lse = np.empty((B, H_q, chunks))
    _check(_load().tsd_oracle_sparse_attention(
        B, H_q, H_kv, D, H_sel, k, chunks, _ptr(qc), DTYPE[q_enc], _ptr(kc),
        _ptr(vc), DTYPE[kv_enc], _ptr(ks), _ptr(vs), _ptr(pt), pt.shape[1],
        _ptr(sl), num_pages, page_size, _ptr(ix), _ptr(ct), scale, _ptr(o),
        _ptr(lse)))
    return o, lse


def lse_merge(o_part, lse_part):
    """Merge [rows, C, D] partials -> (out [rows, D], lse [rows])."""
    op = _c(o_part, np.float64)
    lp = _c(lse_part, np.float64)
    C, D = op.shape[-2], op.shape[-1]
    rows = int(np.prod(op.shape[:-2])) if op.ndim > 2 else 1
    out = np.empty((rows, D))
    out_lse = np.empty(rows)
    _check(_load().tsd_oracle_lse_merge(_ptr(op), _ptr(lp), rows, C, D,
                                        _ptr(out), _ptr(out_lse)))
    return out, out_lse


def dense_attention(q, q_enc, k_pool, v_pool, kv_enc, k_scale, v_scale,
                    page_table, seq_lens, num_pages, softmax_scale=None,
                    page_size=64):
    """Dense attention over all cached tokens -> (out [B,H_q,D], lse [B,H_q])."""
    B, H_q, D = q.shape
    H_kv = k_pool.shape[1]
    qc = _codes(q, q_enc)
    kc, vc = _codes(k_pool, kv_enc), _codes(v_pool, kv_enc)
    ks = None if k_scale is None else _c(k_scale, np.float32)
    vs = None if v_scale is None else _c(v_scale, np.float32)
    pt, sl = _c(page_table, np.int32), _c(seq_lens, np.int32)
    scale = softmax_scale if softmax_scale is not None else 1.0 / np.sqrt(D)
    out = np.empty((B, H_q, D))
    out_lse = np.empty((B, H_q))
    _check(_load().tsd_oracle_dense_attention(
        B, H_q, H_kv, D, _ptr(qc), DTYPE[q_enc], _ptr(kc), _ptr(vc),
        DTYPE[kv_enc], _ptr(ks), _ptr(vs), _ptr(pt), pt.shape[1], _ptr(sl),
        num_pages, page_size, scale, _ptr(out), _ptr(out_lse)))
    return out, out_lse


def decode_step(wl, chunks=None):
    """The whole path on the CPU for a host-side workload dict (see
    ``tsd_synth.to_host``): scores -> f32 -> top-k -> chunked attention ->
    merge. Returns a dict of every intermediate."""
    k = wl["top_k"]
    C = chunks or wl["chunks"]
    if wl["mode"] == "ds":
        s64 = ds_scores(wl["q"], wl["q_enc"], wl["channel_idx"],
                        wl["label_pool"], wl["kv_enc"], wl["page_table"],
                        wl["seq_lens"], wl["num_pages"])
        H_kv = wl["channel_idx"].shape[0]
        row_lens = np.repeat(wl["seq_lens"], H_kv)
        H_sel = H_kv
    else:
        s64 = qsa_scores(wl["index_q"], wl["index_w"], wl["index_k"],
                         wl["page_table"], wl["seq_lens"], wl["num_pages"])
        row_lens = wl["seq_lens"]
        H_sel = 1
    s32 = s64.astype(np.float32)
    idx, cnt = topk(s32, row_lens, k)
    B = wl["q"].shape[0]
    idx3 = idx.reshape(B, H_sel, k)
    cnt2 = cnt.reshape(B, H_sel)
    o, lse = sparse_attention(wl["q"], wl["q_enc"], wl["k_pool"], wl["v_pool"],
                              wl["kv_enc"], wl.get("k_scale"),
                              wl.get("v_scale"), wl["page_table"],
                              wl["seq_lens"], wl["num_pages"], idx3, cnt2, C)
    H_q, D = wl["q"].shape[1], wl["q"].shape[2]
    out, out_lse = lse_merge(o.reshape(B * H_q, C, D), lse.reshape(B * H_q, C))
    return {"scores64": s64, "scores32": s32, "row_lens": row_lens,
            "idx": idx3, "count": cnt2, "o_part": o, "lse_part": lse,
            "out": out.reshape(B, H_q, D), "out_lse": out_lse.reshape(B, H_q)}
