"""One decode step of the whole path with preallocated buffers:
sparse_index_score -> topk_select -> sparse_gqa_decode -> lse_merge.

A *layer* is a dict of device tensors and sizes with these keys:
  mode ("ds" | "qsa"), B, H_q, H_kv, D, top_k, chunks, num_pages,
  page_table, seq_lens, q, k_pool, v_pool, k_scale, v_scale (FP8 only),
  ds:  channel_idx, label_pool
  qsa: index_q, index_w, index_k_pool (or index_k), rows_per_req, q_pos.
Buffers are allocated once by ``StepBuffers`` and reused by every call, so a
step allocates nothing.
"""
from __future__ import annotations

import torch

from . import (lse_merge, sparse_gqa_decode, sparse_index_score,
               sparse_index_topk, topk_select, topk_select_workspace_bytes)


class StepBuffers:
    def __init__(self, layer, max_len=None, device="cuda"):
        B, H_q, H_kv, D = layer["B"], layer["H_q"], layer["H_kv"], layer["D"]
        k, C = layer["top_k"], layer["chunks"]
        self.mode = layer["mode"]
        if max_len is None:
            max_len = layer["page_table"].shape[1] * 64
        self.max_len = int(max_len)
        if self.mode == "ds":
            self.rows, self.H_sel = B * H_kv, H_kv
        else:
            self.rows = B * layer.get("rows_per_req", 1)
            self.H_sel = 1
        dev = torch.device(device)
        self.scores = torch.empty((self.rows, self.max_len), dtype=torch.float32,
                                  device=dev)
        self.row_lens = torch.empty(self.rows, dtype=torch.int32, device=dev)
        self.idx = torch.empty((self.rows, k), dtype=torch.int32, device=dev)
        self.count = torch.empty(self.rows, dtype=torch.int32, device=dev)
        # zero-filled once: every selection leaves its histograms zero, so
        # the calls below skip the clearing launch
        self.ws = torch.zeros(
            max(1, topk_select_workspace_bytes(self.rows, self.max_len, k)),
            dtype=torch.uint8, device=dev)
        self.o_part = torch.empty((B, H_q, C, D), dtype=torch.float32, device=dev)
        self.lse_part = torch.empty((B, H_q, C), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, H_q, D), dtype=torch.float32, device=dev)
        self.out_lse = torch.empty((B, H_q), dtype=torch.float32, device=dev)


def score(layer, bufs, stream=None):
    if layer["mode"] == "ds":
        sparse_index_score("ds", bufs.scores, layer["page_table"],
                           layer["seq_lens"], layer["num_pages"], q=layer["q"],
                           channel_idx=layer["channel_idx"],
                           label_pool=layer["label_pool"],
                           row_lens_out=bufs.row_lens, stream=stream)
    else:
        sparse_index_score("qsa", bufs.scores, layer["page_table"],
                           layer["seq_lens"], layer["num_pages"],
                           index_q=layer["index_q"], index_w=layer["index_w"],
                           index_k_pool=layer.get("index_k_pool",
                                                  layer.get("index_k")),
                           q_pos=layer.get("q_pos"),
                           rows_per_req=layer.get("rows_per_req", 1),
                           row_lens_out=bufs.row_lens, stream=stream)


def score_select(layer, bufs, stream=None):
    """sparse_index_topk: the scores and the selection in one call."""
    kw = dict(q_pos=layer.get("q_pos"), rows_per_req=layer.get("rows_per_req", 1),
              stream=stream)
    if layer["mode"] == "ds":
        kw.update(q=layer["q"], channel_idx=layer["channel_idx"],
                  label_pool=layer["label_pool"])
    else:
        kw.update(index_q=layer["index_q"], index_w=layer["index_w"],
                  index_k_pool=layer.get("index_k_pool", layer.get("index_k")))
    sparse_index_topk(layer["mode"], bufs.scores, layer["page_table"],
                      layer["seq_lens"], layer["num_pages"], layer["top_k"],
                      bufs.idx, bufs.count, bufs.ws, bufs.row_lens,
                      ws_zeroed=True, **kw)


def select(layer, bufs, stream=None):
    topk_select(bufs.scores, bufs.row_lens, layer["top_k"], bufs.max_len,
                bufs.idx, bufs.count, bufs.ws, ws_zeroed=True, stream=stream)


def attend(layer, bufs, stream=None):
    B, k = layer["B"], layer["top_k"]
    sparse_gqa_decode(layer["q"], layer["k_pool"], layer["v_pool"],
                      layer["page_table"], layer["seq_lens"],
                      layer["num_pages"], bufs.idx.view(B, bufs.H_sel, k),
                      bufs.count.view(B, bufs.H_sel), layer["chunks"],
                      bufs.o_part, bufs.lse_part, k_scale=layer.get("k_scale"),
                      v_scale=layer.get("v_scale"),
                      dense_len=layer.get("dense_len", 0), stream=stream)


def merge(layer, bufs, stream=None):
    lse_merge(bufs.o_part, bufs.lse_part, bufs.out, bufs.out_lse, stream=stream)


def decode_step(layer, bufs, stream=None, fused=False):
    """All four calls, asynchronously on ``stream`` (default: current);
    ``fused`` replaces the first two with sparse_index_topk."""
    if fused:
        score_select(layer, bufs, stream)
    else:
        score(layer, bufs, stream)
        select(layer, bufs, stream)
    attend(layer, bufs, stream)
    merge(layer, bufs, stream)


class Plan:
    """The C calls of one layer's step with their arguments marshalled once.

    ``run(stream)`` issues sparse_index_score + topk_select (or, with
    ``fused``, sparse_index_topk), then sparse_gqa_decode and lse_merge,
    straight through the C ABI on ``stream`` (a torch stream), so repeated
    steps pay only the foreign-call cost. Per-call hooks (``before`` /
    ``after``, called with the call's name) let a caller bracket individual
    calls with events on the same stream."""

    def __init__(self, layer, bufs, fused=False):
        self.fused = fused
        import ctypes

        from . import (ABI_VERSION, PAGE_SIZE, AttnArgs, ScoreArgs,
                       TSD_SCORE_DS_LABEL, TSD_SCORE_QSA_INDEX,
                       TSD_TOPK_WS_ZEROED, _half_code,
                       _kv_code, _lib)
        P = ctypes.c_void_p
        p = lambda t: None if t is None else P(t.data_ptr())  # noqa: E731
        self._lib, self._keep = _lib, (layer, bufs)
        a = ScoreArgs()
        a.abi_version, a.page_size = ABI_VERSION, PAGE_SIZE
        a.B = layer["page_table"].shape[0]
        a.page_table, a.pt_stride = p(layer["page_table"]), layer["page_table"].shape[1]
        a.seq_lens, a.num_pages = p(layer["seq_lens"]), int(layer["num_pages"])
        a.scores, a.score_stride = p(bufs.scores), bufs.scores.shape[-1]
        a.row_lens_out = p(bufs.row_lens)
        if layer["mode"] == "ds":
            a.mode = TSD_SCORE_DS_LABEL
            q = layer["q"]
            a.q, a.q_dtype = p(q), _half_code(q)
            a.H_q, a.D = q.shape[1], q.shape[2]
            a.H_kv, a.r = layer["channel_idx"].shape
            a.channel_idx = p(layer["channel_idx"])
            a.label_pool = p(layer["label_pool"])
            a.label_dtype = _half_code(layer["label_pool"])
        else:
            a.mode = TSD_SCORE_QSA_INDEX
            ik = layer.get("index_k_pool", layer.get("index_k"))
            a.index_q, a.index_w = p(layer["index_q"]), p(layer["index_w"])
            a.index_k_pool, a.q_pos = p(ik), p(layer.get("q_pos"))
            a.rows_per_req = layer.get("rows_per_req", 1)
            a.H_i, a.D_i = layer["index_q"].shape[1], layer["index_q"].shape[2]
        self.score_args = a
        k = layer["top_k"]
        self.topk_args = (p(bufs.scores), bufs.scores.shape[-1], bufs.rows,
                          p(bufs.row_lens), bufs.max_len, k, p(bufs.idx),
                          p(bufs.count), p(bufs.ws), bufs.ws.numel(),
                          TSD_TOPK_WS_ZEROED)
        t = AttnArgs()
        q = layer["q"]
        t.abi_version, t.page_size = ABI_VERSION, PAGE_SIZE
        t.B, t.H_q, t.D = q.shape
        t.H_kv = layer["k_pool"].shape[1]
        t.q, t.q_dtype = p(q), _half_code(q)
        t.k_pool, t.v_pool = p(layer["k_pool"]), p(layer["v_pool"])
        t.kv_dtype = _kv_code(layer["k_pool"])
        t.k_scale, t.v_scale = p(layer.get("k_scale")), p(layer.get("v_scale"))
        t.page_table, t.pt_stride = a.page_table, a.pt_stride
        t.seq_lens, t.num_pages = a.seq_lens, a.num_pages
        t.idx, t.count, t.H_sel, t.k = p(bufs.idx), p(bufs.count), bufs.H_sel, k
        t.chunks = layer["chunks"]
        t.softmax_scale = 1.0 / (t.D ** 0.5)
        t.o_part, t.lse_part = p(bufs.o_part), p(bufs.lse_part)
        self.attn_args = t
        C, D = bufs.o_part.shape[-2], bufs.o_part.shape[-1]
        self.merge_args = (p(bufs.o_part), p(bufs.lse_part),
                           bufs.lse_part.numel() // C, C, D, p(bufs.out),
                           p(bufs.out_lse))
        self._score_ref = ctypes.byref(self.score_args)
        self._attn_ref = ctypes.byref(self.attn_args)

    def calls(self, stream=None):
        """(name, launch) pairs of this plan's C calls on ``stream``."""
        import ctypes
        s = stream if stream is not None else torch.cuda.current_stream()
        h = ctypes.c_void_p(s.cuda_stream)
        lib = self._lib
        if self.fused:
            first = (("sparse_index_topk",
                      lambda: lib.sparse_index_topk(
                          self._score_ref, self.topk_args[5], self.topk_args[6],
                          self.topk_args[7], self.topk_args[8],
                          self.topk_args[9], self.topk_args[10], h)),)
        else:
            first = (("sparse_index_score",
                      lambda: lib.sparse_index_score(self._score_ref, h)),
                     ("topk_select",
                      lambda: lib.topk_select_ex(*self.topk_args, h)))
        return first + (
            ("sparse_gqa_decode", lambda: lib.sparse_gqa_decode(self._attn_ref, h)),
            ("lse_merge", lambda: lib.lse_merge(*self.merge_args, h)))

    def run(self, stream=None, before=None, after=None):
        from . import TsdError
        for name, fn in self.calls(stream):
            if before:
                before(name)
            rc = fn()
            if rc:
                raise TsdError(name, rc)
            if after:
                after(name)
