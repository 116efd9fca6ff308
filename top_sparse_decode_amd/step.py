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

from . import (lse_merge, sparse_gqa_decode, sparse_index_score, topk_select,
               topk_select_workspace_bytes)


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
        self.ws = torch.empty(
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


def select(layer, bufs, stream=None):
    topk_select(bufs.scores, bufs.row_lens, layer["top_k"], bufs.max_len,
                bufs.idx, bufs.count, bufs.ws, stream=stream)


def attend(layer, bufs, stream=None):
    B, k = layer["B"], layer["top_k"]
    sparse_gqa_decode(layer["q"], layer["k_pool"], layer["v_pool"],
                      layer["page_table"], layer["seq_lens"],
                      layer["num_pages"], bufs.idx.view(B, bufs.H_sel, k),
                      bufs.count.view(B, bufs.H_sel), layer["chunks"],
                      bufs.o_part, bufs.lse_part, k_scale=layer.get("k_scale"),
                      v_scale=layer.get("v_scale"), stream=stream)


def merge(layer, bufs, stream=None):
    lse_merge(bufs.o_part, bufs.lse_part, bufs.out, bufs.out_lse, stream=stream)


def decode_step(layer, bufs, stream=None):
    """All four calls, asynchronously on ``stream`` (default: current)."""
    score(layer, bufs, stream)
    select(layer, bufs, stream)
    attend(layer, bufs, stream)
    merge(layer, bufs, stream)
