"""Python binding of libtsd.so (top-k sparse decode attention for MI355X).

Argument marshalling only: every function checks tensor placement, dtype and
contiguity, then calls the C entry point of the same name on the current HIP
stream (or the one given). All compute runs in the library's gfx950 kernels;
there is no fallback of any kind, and importing this package raises when the
built library is missing. Outputs are caller-allocated tensors, so the calls
allocate nothing and can be captured in a HIP graph.

Stored encodings: bf16 / fp16 tensors as such; FP8 E4M3 tensors either as
``torch.float8_e4m3fn`` or as their ``uint8`` codes.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

from . import _srchash

_PKG = os.path.dirname(os.path.abspath(__file__))
# TSD_LIB names another build of the same sources (the tests' host-sanitizer
# build); it must still carry the digest of the sources beside it.
LIB_PATH = os.environ.get("TSD_LIB") or os.path.join(_PKG, "libtsd.so")

TSD_BF16, TSD_FP16, TSD_FP8_E4M3, TSD_F32 = 1, 2, 3, 4
TSD_SCORE_DS_LABEL, TSD_SCORE_QSA_INDEX = 1, 2
TSD_TOPK_WS_ZEROED = 1
ABI_VERSION = 1
PAGE_SIZE = 64

_P, _I32, _I64, _F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float


class ScoreArgs(ctypes.Structure):
    _fields_ = [
        ("abi_version", _I32), ("mode", _I32), ("B", _I32), ("page_size", _I32),
        ("page_table", _P), ("pt_stride", _I64), ("seq_lens", _P),
        ("num_pages", _I64),
        ("q", _P), ("q_dtype", _I32), ("H_q", _I32), ("H_kv", _I32),
        ("D", _I32), ("channel_idx", _P), ("r", _I32), ("label_dtype", _I32),
        ("label_pool", _P),
        ("index_q", _P), ("index_w", _P), ("index_k_pool", _P), ("q_pos", _P),
        ("rows_per_req", _I32), ("H_i", _I32), ("D_i", _I32),
        ("reserved0", _I32),
        ("scores", _P), ("score_stride", _I64), ("row_lens_out", _P),
    ]


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("abi_version", _I32), ("B", _I32), ("H_q", _I32), ("H_kv", _I32),
        ("D", _I32), ("q_dtype", _I32), ("q", _P), ("k_pool", _P),
        ("v_pool", _P), ("kv_dtype", _I32), ("page_size", _I32),
        ("k_scale", _P), ("v_scale", _P), ("page_table", _P),
        ("pt_stride", _I64), ("seq_lens", _P), ("num_pages", _I64),
        ("idx", _P), ("count", _P), ("H_sel", _I32), ("k", _I32),
        ("chunks", _I32), ("softmax_scale", _F32), ("o_part", _P),
        ("lse_part", _P), ("dense_len", _I32), ("idx_block", _I32),
    ]


class AppendArgs(ctypes.Structure):
    _fields_ = [
        ("abi_version", _I32), ("B", _I32), ("page_size", _I32),
        ("max_new", _I32), ("page_table", _P), ("pt_stride", _I64),
        ("num_pages", _I64), ("positions", _P), ("n_new", _P),
        ("H_kv", _I32), ("D", _I32), ("new_dtype", _I32), ("kv_dtype", _I32),
        ("k_new", _P), ("v_new", _P), ("k_pool", _P), ("v_pool", _P),
        ("k_scale", _P), ("v_scale", _P), ("channel_idx", _P),
        ("label_pool", _P), ("r", _I32), ("index_dtype", _I32),
        ("index_k_new", _P), ("index_k_pool", _P), ("D_i", _I32),
        ("reserved0", _I32),
    ]


class CompressArgs(ctypes.Structure):
    _fields_ = [
        ("abi_version", _I32), ("B", _I32), ("page_size", _I32),
        ("block_size", _I32), ("index_k_pool", _P), ("page_table", _P),
        ("pt_stride", _I64), ("num_pages", _I64), ("seq_lens", _P),
        ("from_block", _P), ("max_blocks", _I32), ("D_i", _I32),
        ("ck_pool", _P), ("cpage_table", _P), ("cpt_stride", _I64),
        ("num_cpages", _I64),
    ]


class TsdError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {_lib.tsd_strerror(status).decode()} "
                         f"(status {status})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python top_sparse_decode_amd/build_lib.py)")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "sparse_index_score": (ctypes.c_int, [ctypes.POINTER(ScoreArgs), _P]),
        "topk_select_workspace_bytes": (ctypes.c_size_t,
                                        [ctypes.c_int, ctypes.c_int, ctypes.c_int]),
        "topk_select": (ctypes.c_int, [_P, _I64, ctypes.c_int, _P, ctypes.c_int,
                                       ctypes.c_int, _P, _P, _P,
                                       ctypes.c_size_t, _P]),
        "topk_select_ex": (ctypes.c_int, [_P, _I64, ctypes.c_int, _P,
                                          ctypes.c_int, ctypes.c_int, _P, _P,
                                          _P, ctypes.c_size_t, ctypes.c_int,
                                          _P]),
        "topk_select_noalloc": (ctypes.c_int, [_P, _I64, ctypes.c_int, _P,
                                               ctypes.c_int, ctypes.c_int, _P,
                                               _P, _P]),
        "topk_select_noalloc_max_bytes": (ctypes.c_size_t, []),
        "sparse_index_topk": (ctypes.c_int, [ctypes.POINTER(ScoreArgs),
                                             ctypes.c_int, _P, _P, _P,
                                             ctypes.c_size_t, ctypes.c_int, _P]),
        "topk_merge_sharded": (ctypes.c_int, [_P, _I64, _P, _P, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, _P, _P, _P]),
        "sparse_gqa_decode": (ctypes.c_int, [ctypes.POINTER(AttnArgs), _P]),
        "kv_append": (ctypes.c_int, [ctypes.POINTER(AppendArgs), _P]),
        "index_k_compress": (ctypes.c_int, [ctypes.POINTER(CompressArgs), _P]),
        "expand_blocks": (ctypes.c_int, [_P, _P, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, _P, ctypes.c_int, _P,
                                         _P, _P]),
        "tsd_sizeof_compress_args": (ctypes.c_size_t, []),
        "tsd_sizeof_append_args": (ctypes.c_size_t, []),
        "lse_merge": (ctypes.c_int, [_P, _P, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, _P, _P, _P]),
        "tsd_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "tsd_abi_version": (ctypes.c_int, []),
        "tsd_source_sha256": (ctypes.c_char_p, []),
        "tsd_sizeof_score_args": (ctypes.c_size_t, []),
        "tsd_sizeof_attn_args": (ctypes.c_size_t, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    if lib.tsd_abi_version() != ABI_VERSION:
        raise ImportError("libtsd.so ABI version mismatch")
    if (lib.tsd_sizeof_score_args() != ctypes.sizeof(ScoreArgs)
            or lib.tsd_sizeof_attn_args() != ctypes.sizeof(AttnArgs)
            or lib.tsd_sizeof_append_args() != ctypes.sizeof(AppendArgs)
            or lib.tsd_sizeof_compress_args() != ctypes.sizeof(CompressArgs)):
        raise ImportError("libtsd.so argument struct layout mismatch")
    want = _srchash.source_sha256()
    have = lib.tsd_source_sha256().decode()
    if want is not None and have != want:
        raise ImportError(
            f"{LIB_PATH} was built from other sources than the ones beside it "
            f"(library {have[:16]}, sources {want[:16]}): rebuild it "
            "(python top_sparse_decode_amd/build_lib.py)")
    return lib


_lib = _load()
EXPORTS = ("sparse_index_score", "sparse_index_topk",
           "topk_select_workspace_bytes", "topk_select", "topk_select_ex",
           "topk_select_noalloc", "topk_select_noalloc_max_bytes",
           "topk_merge_sharded", "sparse_gqa_decode", "lse_merge",
           "kv_append", "index_k_compress", "expand_blocks", "tsd_strerror",
           "tsd_abi_version", "tsd_source_sha256",
           "tsd_sizeof_score_args", "tsd_sizeof_attn_args",
           "tsd_sizeof_append_args", "tsd_sizeof_compress_args")


# ----------------------------------------------------------------- helpers
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(name, t, dtype=None, dtypes=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {dtypes}, got {t.dtype}")
    return t


def _shape(name, t, *dims):
    """``t`` (if given) has exactly len(dims) dimensions, each equal to the
    given size where one is given (None: any)."""
    if t is None:
        return t
    shp = tuple(t.shape)
    if len(shp) != len(dims) or any(d is not None and int(d) != s
                                    for d, s in zip(dims, shp)):
        want = "[" + ", ".join("*" if d is None else str(int(d)) for d in dims) + "]"
        raise ValueError(f"{name} has shape {list(shp)}, expected {want}")
    return t


def _pool_rows(name, t, num_pages):
    """A slot-addressed pool holds at least num_pages * 64 slots."""
    if t is not None and t.shape[0] < int(num_pages) * PAGE_SIZE:
        raise ValueError(f"{name} has {t.shape[0]} slots, fewer than "
                         f"num_pages * 64 = {int(num_pages) * PAGE_SIZE}")


def _page_vec(name, t, num_pages):
    if t is not None and (t.dim() != 1 or t.shape[0] < int(num_pages)):
        raise ValueError(f"{name} must hold one value per page "
                         f"(>= {int(num_pages)}), got shape {list(t.shape)}")


def _half_code(t):
    return {torch.bfloat16: TSD_BF16, torch.float16: TSD_FP16}[t.dtype]


def _kv_code(t):
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return TSD_FP8_E4M3
    return _half_code(t)


_FP8 = (torch.uint8, torch.float8_e4m3fn)
_HALF = (torch.bfloat16, torch.float16)


def _check(fn, rc):
    if rc != 0:
        raise TsdError(fn, rc)


# --------------------------------------------------------------- entry points
def _batch_view(page_table, seq_lens):
    _shape("page_table", page_table, None, None)
    B = page_table.shape[0]
    _shape("seq_lens", seq_lens, B)
    return B


def _score_args(mode, scores, page_table, seq_lens, num_pages, q, channel_idx,
                label_pool, index_q, index_w, index_k_pool, q_pos,
                rows_per_req, row_lens_out):
    B = _batch_view(page_table, seq_lens)
    _shape("scores", scores, None, None)
    if mode == "ds":
        _shape("q", q, B, None, None)
        _shape("channel_idx", channel_idx, None, None)
        H_kv, r = channel_idx.shape
        _shape("label_pool", label_pool, None, H_kv, r)
        _pool_rows("label_pool", label_pool, num_pages)
        rows = B * H_kv
    elif mode == "qsa":
        rows = B * int(rows_per_req)
        _shape("index_q", index_q, rows, None, None)
        _shape("index_w", index_w, rows, index_q.shape[1])
        _shape("index_k_pool", index_k_pool, None, index_q.shape[2])
        _pool_rows("index_k_pool", index_k_pool, num_pages)
        _shape("q_pos", q_pos, rows)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    _shape("scores", scores, rows, None)
    _shape("row_lens_out", row_lens_out, rows)
    _dev("scores", scores, torch.float32)
    _dev("page_table", page_table, torch.int32)
    _dev("seq_lens", seq_lens, torch.int32)
    a = ScoreArgs()
    a.abi_version, a.page_size = ABI_VERSION, PAGE_SIZE
    a.B = B
    a.page_table, a.pt_stride = _ptr(page_table), page_table.shape[1]
    a.seq_lens, a.num_pages = _ptr(seq_lens), int(num_pages)
    a.scores, a.score_stride = _ptr(scores), scores.shape[-1]
    a.row_lens_out = _ptr(_dev("row_lens_out", row_lens_out, torch.int32))
    if mode == "ds":
        _dev("q", q, dtypes=_HALF)
        _dev("channel_idx", channel_idx, torch.int32)
        _dev("label_pool", label_pool, dtypes=_HALF)
        a.mode = TSD_SCORE_DS_LABEL
        a.q, a.q_dtype = _ptr(q), _half_code(q)
        a.H_q, a.D = q.shape[1], q.shape[2]
        a.H_kv, a.r = channel_idx.shape
        a.channel_idx = _ptr(channel_idx)
        a.label_pool, a.label_dtype = _ptr(label_pool), _half_code(label_pool)
    else:
        _dev("index_q", index_q, dtypes=_FP8)
        _dev("index_w", index_w, torch.float32)
        _dev("index_k_pool", index_k_pool, dtypes=_FP8)
        _dev("q_pos", q_pos, torch.int32)
        a.mode = TSD_SCORE_QSA_INDEX
        a.index_q, a.index_w = _ptr(index_q), _ptr(index_w)
        a.index_k_pool, a.q_pos = _ptr(index_k_pool), _ptr(q_pos)
        a.rows_per_req = int(rows_per_req)
        a.H_i, a.D_i = index_q.shape[1], index_q.shape[2]
    return a, rows


def sparse_index_score(mode, scores, page_table, seq_lens, num_pages, *,
                       q=None, channel_idx=None, label_pool=None,
                       index_q=None, index_w=None, index_k_pool=None,
                       q_pos=None, rows_per_req=1, row_lens_out=None,
                       stream=None):
    """Score every cached token of every row into ``scores`` [rows, stride].

    mode "ds":  q [B,H_q,128] bf16/fp16, channel_idx [H_kv,r] int32,
                label_pool [slots,H_kv,r] (q's dtype); rows = B*H_kv.
    mode "qsa": index_q [rows,H_i,128] fp8, index_w [rows,H_i] f32,
                index_k_pool [slots,128] fp8, q_pos [rows] int32 or None;
                rows = B*rows_per_req.
    ``row_lens_out`` (int32 [rows], optional) receives each row's key count.
    """
    a, _ = _score_args(mode, scores, page_table, seq_lens, num_pages, q,
                       channel_idx, label_pool, index_q, index_w,
                       index_k_pool, q_pos, rows_per_req, row_lens_out)
    _check("sparse_index_score", _lib.sparse_index_score(ctypes.byref(a),
                                                         _stream(stream)))


def sparse_index_topk(mode, scores, page_table, seq_lens, num_pages, k, idx,
                      count, workspace, row_lens_out, *, q=None,
                      channel_idx=None, label_pool=None, index_q=None,
                      index_w=None, index_k_pool=None, q_pos=None,
                      rows_per_req=1, ws_zeroed=False, stream=None):
    """sparse_index_score then topk_select on its scores (same results, fewer
    passes). ``row_lens_out`` is required; ``workspace`` and ``ws_zeroed`` as
    for topk_select with max_len = min(scores.shape[-1],
    page_table.shape[1] * 64)."""
    if row_lens_out is None:
        raise ValueError("sparse_index_topk needs row_lens_out")
    _shape("page_table", page_table, None, None)
    if mode == "ds":
        _shape("channel_idx", channel_idx, None, None)
        rows = page_table.shape[0] * channel_idx.shape[0]
    else:
        rows = page_table.shape[0] * int(rows_per_req)
    _shape("idx", idx, rows, k)
    _shape("count", count, rows)
    a, _ = _score_args(mode, scores, page_table, seq_lens, num_pages, q,
                       channel_idx, label_pool, index_q, index_w,
                       index_k_pool, q_pos, rows_per_req, row_lens_out)
    _dev("idx", idx, torch.int32)
    _dev("count", count, torch.int32)
    _dev("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("sparse_index_topk", _lib.sparse_index_topk(
        ctypes.byref(a), int(k), _ptr(idx), _ptr(count), _ptr(workspace),
        ws_bytes, TSD_TOPK_WS_ZEROED if ws_zeroed else 0, _stream(stream)))


def topk_select_workspace_bytes(rows, max_len, k):
    return int(_lib.topk_select_workspace_bytes(int(rows), int(max_len), int(k)))


def topk_select(scores, row_lens, k, max_len, idx, count=None, workspace=None,
                ws_zeroed=False, stream=None):
    """Exact top-k per row of ``scores`` [rows, stride] into ``idx`` [rows, k]
    (ascending, -1 padded) and ``count`` [rows]. ``workspace`` is a uint8
    CUDA tensor of at least topk_select_workspace_bytes(rows, max_len, k).
    ``ws_zeroed``: its histogram words are zero already (zero-filled, or last
    used by a call with at least as many rows), so the call goes through
    topk_select_ex with TSD_TOPK_WS_ZEROED and skips the clearing launch;
    every call leaves them zero."""
    _shape("scores", scores, None, None)
    rows = scores.shape[0]
    _shape("row_lens", row_lens, rows)
    _shape("idx", idx, rows, k)
    _shape("count", count, rows)
    _dev("scores", scores, torch.float32)
    _dev("row_lens", row_lens, torch.int32)
    _dev("idx", idx, torch.int32)
    _dev("count", count, torch.int32)
    _dev("workspace", workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(scores), scores.shape[-1], rows, _ptr(row_lens), int(max_len),
            int(k), _ptr(idx), _ptr(count), _ptr(workspace), ws_bytes)
    if ws_zeroed:
        _check("topk_select_ex", _lib.topk_select_ex(
            *args, TSD_TOPK_WS_ZEROED, _stream(stream)))
    else:
        _check("topk_select", _lib.topk_select(*args, _stream(stream)))


def topk_select_noalloc(scores, row_lens, k, max_len, idx, count=None,
                        stream=None):
    """topk_select without a caller workspace: the library's fixed device
    scratch (topk_select_noalloc_max_bytes(), shared by every call on the
    GPU) holds it, so nothing is allocated; calls on one GPU must not
    overlap."""
    _shape("scores", scores, None, None)
    rows = scores.shape[0]
    _shape("row_lens", row_lens, rows)
    _shape("idx", idx, rows, k)
    _shape("count", count, rows)
    _dev("scores", scores, torch.float32)
    _dev("row_lens", row_lens, torch.int32)
    _dev("idx", idx, torch.int32)
    _dev("count", count, torch.int32)
    _check("topk_select_noalloc", _lib.topk_select_noalloc(
        _ptr(scores), scores.shape[-1], rows, _ptr(row_lens), int(max_len),
        int(k), _ptr(idx), _ptr(count), _stream(stream)))


def topk_merge_sharded(scores, idx_local, count_local, k, idx, count=None,
                       stream=None):
    """Exact global top-k from W page-owner shards: ``scores`` [W, rows,
    stride] (shard-local order), ``idx_local`` [W, rows, kl] and
    ``count_local`` [W, rows] (each shard's topk_select output) into ``idx``
    [rows, k] (ascending global tokens, -1 padded) and ``count`` [rows]."""
    _shape("scores", scores, None, None, None)
    W, rows, stride = scores.shape
    _shape("idx_local", idx_local, W, rows, None)
    _shape("count_local", count_local, W, rows)
    _shape("idx", idx, rows, k)
    _shape("count", count, rows)
    _dev("scores", scores, torch.float32)
    _dev("idx_local", idx_local, torch.int32)
    _dev("count_local", count_local, torch.int32)
    _dev("idx", idx, torch.int32)
    _dev("count", count, torch.int32)
    _check("topk_merge_sharded", _lib.topk_merge_sharded(
        _ptr(scores), stride, _ptr(idx_local), _ptr(count_local), W, rows,
        idx_local.shape[2], int(k), _ptr(idx), _ptr(count), _stream(stream)))


def sparse_gqa_decode(q, k_pool, v_pool, page_table, seq_lens, num_pages, idx,
                      count, chunks, o_part, lse_part, k_scale=None,
                      v_scale=None, softmax_scale=None, dense_len=0,
                      idx_block=0, stream=None):
    """Chunked sparse GQA attention over the selection ``idx`` [B,H_sel,k]
    into ``o_part`` [B,H_q,chunks,128] and ``lse_part`` [B,H_q,chunks].
    ``idx_block`` > 1: ``idx`` holds ascending indices of selected blocks of
    that many tokens (``count`` = blocks) instead of token indices."""
    B = _batch_view(page_table, seq_lens)
    _shape("q", q, B, None, None)
    H_q, D = q.shape[1], q.shape[2]
    _shape("k_pool", k_pool, None, None, D)
    _shape("v_pool", v_pool, *k_pool.shape)
    _pool_rows("k_pool", k_pool, num_pages)
    _page_vec("k_scale", k_scale, num_pages)
    _page_vec("v_scale", v_scale, num_pages)
    _shape("idx", idx, B, None, None)
    _shape("count", count, B, idx.shape[1])
    _shape("o_part", o_part, B, H_q, chunks, D)
    _shape("lse_part", lse_part, B, H_q, chunks)
    _dev("q", q, dtypes=_HALF)
    _dev("k_pool", k_pool, dtypes=_HALF + _FP8)
    _dev("v_pool", v_pool, dtypes=_HALF + _FP8)
    _dev("page_table", page_table, torch.int32)
    _dev("seq_lens", seq_lens, torch.int32)
    _dev("idx", idx, torch.int32)
    _dev("count", count, torch.int32)
    _dev("o_part", o_part, torch.float32)
    _dev("lse_part", lse_part, torch.float32)
    _dev("k_scale", k_scale, torch.float32)
    _dev("v_scale", v_scale, torch.float32)
    a = AttnArgs()
    a.abi_version, a.page_size = ABI_VERSION, PAGE_SIZE
    a.B, a.H_q, a.D = q.shape
    a.H_kv = k_pool.shape[1]
    a.q, a.q_dtype = _ptr(q), _half_code(q)
    a.k_pool, a.v_pool, a.kv_dtype = _ptr(k_pool), _ptr(v_pool), _kv_code(k_pool)
    a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    a.page_table, a.pt_stride = _ptr(page_table), page_table.shape[1]
    a.seq_lens, a.num_pages = _ptr(seq_lens), int(num_pages)
    a.idx, a.count = _ptr(idx), _ptr(count)
    a.H_sel, a.k = idx.shape[1], idx.shape[2]
    a.chunks = int(chunks)
    a.softmax_scale = (1.0 / math.sqrt(a.D) if softmax_scale is None
                       else float(softmax_scale))
    a.o_part, a.lse_part = _ptr(o_part), _ptr(lse_part)
    a.dense_len = int(dense_len)
    a.idx_block = int(idx_block)
    _check("sparse_gqa_decode", _lib.sparse_gqa_decode(ctypes.byref(a),
                                                       _stream(stream)))


def kv_append(page_table, num_pages, positions, n_new, max_new, *,
              k_new=None, v_new=None, k_pool=None, v_pool=None, k_scale=None,
              v_scale=None, channel_idx=None, label_pool=None,
              index_k_new=None, index_k_pool=None, stream=None,
              prepare=False):
    """Store new tokens' rows: ``k_new``/``v_new`` [B, max_new, H_kv, 128]
    (bf16/fp16) into ``k_pool``/``v_pool`` (same encoding, or FP8 with
    ``k_scale``/``v_scale`` [num_pages]); the label rows K[channel_idx] into
    ``label_pool``; ``index_k_new`` [B, max_new, 128] (bf16/fp16/f32) into
    the FP8 ``index_k_pool``. Token positions[b] + i, i < n_new[b].
    With ``prepare=True`` nothing is launched: the marshalled call is
    returned as a function of no arguments (it returns the C status)."""
    _shape("page_table", page_table, None, None)
    B = page_table.shape[0]
    _shape("positions", positions, B)
    _shape("n_new", n_new, B)
    if k_pool is not None or channel_idx is not None:
        if k_new is None:
            raise ValueError("k_new is required with k_pool or channel_idx")
        _shape("k_new", k_new, B, max_new, None, None)
        H_kv, D = k_new.shape[2], k_new.shape[3]
    if k_pool is not None:
        if v_new is None or v_pool is None:
            raise ValueError("v_new and v_pool go with k_pool")
        _shape("v_new", v_new, *k_new.shape)
        _shape("k_pool", k_pool, None, H_kv, D)
        _shape("v_pool", v_pool, *k_pool.shape)
        _pool_rows("k_pool", k_pool, num_pages)
        _page_vec("k_scale", k_scale, num_pages)
        _page_vec("v_scale", v_scale, num_pages)
    if channel_idx is not None:
        _shape("channel_idx", channel_idx, H_kv, None)
        _shape("label_pool", label_pool, None, H_kv, channel_idx.shape[1])
        _pool_rows("label_pool", label_pool, num_pages)
    if index_k_new is not None:
        _shape("index_k_new", index_k_new, B, max_new, None)
        _shape("index_k_pool", index_k_pool, None, index_k_new.shape[2])
        _pool_rows("index_k_pool", index_k_pool, num_pages)
    _dev("page_table", page_table, torch.int32)
    _dev("positions", positions, torch.int32)
    _dev("n_new", n_new, torch.int32)
    _dev("k_new", k_new, dtypes=_HALF)
    _dev("v_new", v_new, dtypes=_HALF)
    _dev("k_pool", k_pool, dtypes=_HALF + _FP8)
    _dev("v_pool", v_pool, dtypes=_HALF + _FP8)
    _dev("k_scale", k_scale, torch.float32)
    _dev("v_scale", v_scale, torch.float32)
    _dev("channel_idx", channel_idx, torch.int32)
    _dev("label_pool", label_pool, dtypes=_HALF)
    _dev("index_k_new", index_k_new, dtypes=_HALF + (torch.float32,))
    _dev("index_k_pool", index_k_pool, dtypes=_FP8)
    a = AppendArgs()
    a.abi_version, a.page_size = ABI_VERSION, PAGE_SIZE
    a.B, a.max_new = B, int(max_new)
    a.page_table, a.pt_stride = _ptr(page_table), page_table.shape[1]
    a.num_pages = int(num_pages)
    a.positions, a.n_new = _ptr(positions), _ptr(n_new)
    if k_new is not None:
        a.H_kv, a.D = k_new.shape[2], k_new.shape[3]
        a.new_dtype = _half_code(k_new)
    if k_pool is not None:
        a.k_new, a.v_new = _ptr(k_new), _ptr(v_new)
        a.k_pool, a.v_pool, a.kv_dtype = _ptr(k_pool), _ptr(v_pool), _kv_code(k_pool)
        a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    if channel_idx is not None:
        a.k_new = _ptr(k_new)
        a.channel_idx, a.r = _ptr(channel_idx), channel_idx.shape[1]
        a.label_pool = _ptr(label_pool)
    if index_k_new is not None:
        a.index_k_new, a.index_k_pool = _ptr(index_k_new), _ptr(index_k_pool)
        a.index_dtype = (TSD_F32 if index_k_new.dtype == torch.float32
                         else _half_code(index_k_new))
        a.D_i = index_k_new.shape[2]
    if prepare:
        st = _stream(stream)
        ref = ctypes.byref(a)
        fn = _lib.kv_append
        keep = (page_table, positions, n_new, k_new, v_new, k_pool, v_pool,
                k_scale, v_scale, channel_idx, label_pool, index_k_new,
                index_k_pool)  # the tensors stay alive with the call
        return lambda keep=keep: fn(ref, st)
    _check("kv_append", _lib.kv_append(ctypes.byref(a), _stream(stream)))


def index_k_compress(index_k_pool, page_table, num_pages, seq_lens,
                     ck_pool, cpage_table, num_cpages, block_size,
                     max_blocks, from_block=None, stream=None):
    """Compressed index keys of blocks [from_block[b], from_block[b] +
    max_blocks) below ceil(seq_lens[b] / block_size) into ``ck_pool``."""
    B = _batch_view(page_table, seq_lens)
    _shape("index_k_pool", index_k_pool, None, None)
    _pool_rows("index_k_pool", index_k_pool, num_pages)
    _shape("from_block", from_block, B)
    _shape("cpage_table", cpage_table, B, None)
    _shape("ck_pool", ck_pool, None, index_k_pool.shape[1])
    _pool_rows("ck_pool", ck_pool, num_cpages)
    _dev("index_k_pool", index_k_pool, dtypes=_FP8)
    _dev("page_table", page_table, torch.int32)
    _dev("seq_lens", seq_lens, torch.int32)
    _dev("from_block", from_block, torch.int32)
    _dev("ck_pool", ck_pool, dtypes=_FP8)
    _dev("cpage_table", cpage_table, torch.int32)
    a = CompressArgs()
    a.abi_version, a.page_size = ABI_VERSION, PAGE_SIZE
    a.B, a.block_size = B, int(block_size)
    a.index_k_pool = _ptr(index_k_pool)
    a.page_table, a.pt_stride = _ptr(page_table), page_table.shape[1]
    a.num_pages, a.seq_lens = int(num_pages), _ptr(seq_lens)
    a.from_block, a.max_blocks = _ptr(from_block), int(max_blocks)
    a.D_i = index_k_pool.shape[1]
    a.ck_pool = _ptr(ck_pool)
    a.cpage_table, a.cpt_stride = _ptr(cpage_table), cpage_table.shape[1]
    a.num_cpages = int(num_cpages)
    _check("index_k_compress", _lib.index_k_compress(ctypes.byref(a),
                                                     _stream(stream)))


def expand_blocks(sel, count, block_size, row_lens, tok, tok_count=None,
                  stream=None):
    """Selected blocks ``sel`` [rows, kb] (first ``count`` [rows]) -> their
    tokens ``tok`` [rows, kt] ascending, -1 padded; ``tok_count`` [rows]."""
    _shape("sel", sel, None, None)
    rows, kb = sel.shape
    _shape("count", count, rows)
    _shape("row_lens", row_lens, rows)
    _shape("tok", tok, rows, None)
    _shape("tok_count", tok_count, rows)
    _dev("sel", sel, torch.int32)
    _dev("count", count, torch.int32)
    _dev("row_lens", row_lens, torch.int32)
    _dev("tok", tok, torch.int32)
    _dev("tok_count", tok_count, torch.int32)
    _check("expand_blocks", _lib.expand_blocks(
        _ptr(sel), _ptr(count), rows, kb, int(block_size), _ptr(row_lens),
        tok.shape[1], _ptr(tok), _ptr(tok_count), _stream(stream)))


def lse_merge(o_part, lse_part, out, out_lse=None, stream=None):
    """Merge ``o_part`` [..., C, D] / ``lse_part`` [..., C] into ``out``
    [..., D] and ``out_lse`` [...]."""
    if o_part.dim() < 2:
        raise ValueError(f"o_part has shape {list(o_part.shape)}, expected "
                         "[..., C, D]")
    lead, (C, D) = tuple(o_part.shape[:-2]), o_part.shape[-2:]
    _shape("lse_part", lse_part, *lead, C)
    _shape("out", out, *lead, D)
    _shape("out_lse", out_lse, *lead)
    _dev("o_part", o_part, torch.float32)
    _dev("lse_part", lse_part, torch.float32)
    _dev("out", out, torch.float32)
    _dev("out_lse", out_lse, torch.float32)
    rows = lse_part.numel() // C if C else 0
    _check("lse_merge", _lib.lse_merge(_ptr(o_part), _ptr(lse_part), rows, C,
                                       D, _ptr(out), _ptr(out_lse),
                                       _stream(stream)))
