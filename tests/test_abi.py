"""The C-ABI library on the host: it loads, exports every function the header
declares, and rejects bad arguments before launching anything. No call here
reaches a kernel, so the file runs without a GPU."""
import ctypes
import os
import re

import pytest

import top_sparse_decode_amd as tsd
from top_sparse_decode_amd import AttnArgs, ScoreArgs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsd.h")
LIB = tsd._lib

E = dict(OK=0, NULL=-1, DTYPE=-2, SHAPE=-3, PAGE_SIZE=-4, GQA=-5, K=-6,
         CHUNKS=-7, WORKSPACE=-8, UNSUPPORTED=-9, MODE=-10, ABI=-11,
         SCRATCH=-12)
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(",
                                 text, flags=re.M)) - {"if"})


def test_header_functions_are_exported():
    names = _declared_functions()
    assert {"sparse_index_score", "topk_select", "sparse_gqa_decode",
            "lse_merge", "topk_select_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(LIB, n), n
        assert n in tsd.EXPORTS


def test_abi_version_and_struct_layout():
    assert LIB.tsd_abi_version() == 1
    assert LIB.tsd_sizeof_score_args() == ctypes.sizeof(ScoreArgs)
    assert LIB.tsd_sizeof_attn_args() == ctypes.sizeof(AttnArgs)
    assert LIB.tsd_sizeof_append_args() == ctypes.sizeof(tsd.AppendArgs)


def test_strerror_names_every_code():
    for code in E.values():
        assert LIB.tsd_strerror(code)
    assert b"HIP" in LIB.tsd_strerror(3)


def _score(**kw):
    a = ScoreArgs()
    a.abi_version, a.mode, a.B, a.page_size = 1, 2, 2, 64
    a.page_table, a.pt_stride, a.seq_lens, a.num_pages = FAKE, 4, FAKE, 8
    a.index_q, a.index_w, a.index_k_pool = FAKE, FAKE, FAKE
    a.rows_per_req, a.H_i, a.D_i = 1, 16, 128
    a.q, a.q_dtype, a.H_q, a.H_kv, a.D = FAKE, 1, 32, 8, 128
    a.channel_idx, a.r, a.label_dtype, a.label_pool = FAKE, 16, 1, FAKE
    a.scores, a.score_stride = FAKE, 256
    for k, v in kw.items():
        setattr(a, k, v)
    return LIB.sparse_index_score(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,code", [
    (dict(abi_version=2), "ABI"),
    (dict(mode=7), "MODE"),
    (dict(page_size=32), "PAGE_SIZE"),
    (dict(B=-1), "SHAPE"),
    (dict(pt_stride=0), "SHAPE"),
    (dict(score_stride=0), "SHAPE"),
    (dict(scores=None), "NULL"),
    (dict(page_table=None), "NULL"),
    (dict(index_k_pool=None), "NULL"),
    (dict(H_i=17), "UNSUPPORTED"),
    (dict(D_i=64), "UNSUPPORTED"),
    (dict(rows_per_req=0), "SHAPE"),
    (dict(mode=1, H_q=30), "GQA"),
    (dict(mode=1, label_dtype=2), "DTYPE"),
    (dict(mode=1, q_dtype=3, label_dtype=3), "DTYPE"),
    (dict(mode=1, D=64), "UNSUPPORTED"),
    (dict(mode=1, r=0), "SHAPE"),
    (dict(mode=1, channel_idx=None), "NULL"),
    (dict(mode=1, H_kv=8, r=1024), "UNSUPPORTED"),
])
def test_score_rejections(kw, code):
    assert _score(**kw) == E[code]


def test_score_null_args_and_empty_batch():
    assert LIB.sparse_index_score(None, None) == E["NULL"]
    # an empty batch is valid and launches nothing
    assert _score(B=0, scores=None, page_table=None, seq_lens=None) == 0


def test_fused_score_topk_rejections():
    def call(k=10, row_lens=True, ws_bytes=None, flags=0, **kw):
        a = ScoreArgs()
        a.abi_version, a.mode, a.B, a.page_size = 1, 2, 2, 64
        a.page_table, a.pt_stride, a.seq_lens, a.num_pages = FAKE, 4, FAKE, 8
        a.index_q, a.index_w, a.index_k_pool = FAKE, FAKE, FAKE
        a.rows_per_req, a.H_i, a.D_i = 1, 16, 128
        a.scores, a.score_stride = FAKE, 256
        a.row_lens_out = FAKE if row_lens else None
        for key, v in kw.items():
            setattr(a, key, v)
        need = LIB.topk_select_workspace_bytes(2, 256, max(1, k))
        return LIB.sparse_index_topk(ctypes.byref(a), k, FAKE, None, FAKE,
                                     need if ws_bytes is None else ws_bytes,
                                     flags, None)
    assert call(row_lens=False) == E["NULL"]
    assert call(k=0) == E["K"]
    assert call(ws_bytes=8) == E["WORKSPACE"]
    assert call(page_size=16) == E["PAGE_SIZE"]
    assert call(B=0, scores=None, page_table=None, seq_lens=None) == 0
    assert call(flags=2) == E["UNSUPPORTED"]


def _topk(rows=2, max_len=100, k=10, stride=128, ws_bytes=None, flags=None,
          **kw):
    """topk_select, or topk_select_ex when flags are given."""
    need = LIB.topk_select_workspace_bytes(rows, max_len, k)
    args = dict(scores=FAKE, row_lens=FAKE, idx=FAKE, ws=FAKE)
    args.update(kw)
    common = (args["scores"], stride, rows, args["row_lens"], max_len, k,
              args["idx"], None, args["ws"],
              need if ws_bytes is None else ws_bytes)
    if flags is None:
        return LIB.topk_select(*common, None)
    return LIB.topk_select_ex(*common, flags, None)


def _prototype(name):
    """Parameter types of a function declared in the public header, with
    the parameter names dropped and spacing normalised."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, name
    out = []
    for p in m.group(1).split(","):
        p = " ".join(p.replace("*", " * ").split())
        out.append(re.sub(r"\s*\w+$", "", p).strip())
    return out


def test_topk_select_prototype_is_the_contract():
    """topk_select takes exactly (scores, stride, rows, row_lens, max_len, k,
    idx, count, ws, ws_bytes, stream); the zeroed-workspace shortcut has a
    name of its own."""
    assert _prototype("topk_select") == [
        "const float *", "int64_t", "int", "const int32_t *", "int", "int",
        "int32_t *", "int32_t *", "void *", "size_t", "hipStream_t"]
    assert _prototype("topk_select_ex") == _prototype("topk_select")[:-1] + [
        "int", "hipStream_t"]
    assert _prototype("sparse_gqa_decode") == ["const tsd_attn_args *",
                                               "hipStream_t"]
    assert _prototype("sparse_index_score") == ["const tsd_score_args *",
                                                "hipStream_t"]
    assert _prototype("lse_merge") == [
        "const float *", "const float *", "int", "int", "int", "float *",
        "float *", "hipStream_t"]


def test_topk_rejections():
    assert _topk(k=0) == E["K"]
    assert _topk(k=4097) == E["K"]
    assert _topk(max_len=200, stride=128) == E["SHAPE"]
    assert _topk(rows=-1) == E["SHAPE"]
    assert _topk(ws_bytes=16) == E["WORKSPACE"]
    assert _topk(ws=None) == E["WORKSPACE"]
    assert _topk(ws=ctypes.c_void_p(0x10008)) == E["WORKSPACE"]  # misaligned
    assert _topk(scores=None) == E["NULL"]
    assert _topk(flags=4) == E["UNSUPPORTED"]
    assert _topk(flags=4, k=0) == E["K"]
    assert _topk(flags=1, ws_bytes=16) == E["WORKSPACE"]
    assert _topk(rows=0, flags=1) == 0
    assert _topk(rows=70000) == E["UNSUPPORTED"]
    assert _topk(max_len=(1 << 24) + 1, stride=(1 << 24) + 1) == E["UNSUPPORTED"]
    assert _topk(rows=0, scores=None, row_lens=None, idx=None, ws=None) == 0


def _ws_words(rows, max_len):
    # 4096- and 1024-bin histograms per row, an 8-byte digit-1 record per
    # row, one counter per 4096-element chunk, padding to 8 bytes, then a
    # 512-entry list of 8-byte pairs per chunk
    nch = max(1, -(-max_len // 4096))
    off = rows * 5120 + rows * 2 + rows * nch
    off += off & 1
    return off + 2 * rows * nch * 512


def test_topk_workspace_size():
    assert tsd.topk_select_workspace_bytes(8, 262144, 2048) == 4 * _ws_words(8, 262144)
    assert tsd.topk_select_workspace_bytes(1, 1, 1) == 4 * _ws_words(1, 1)
    assert tsd.topk_select_workspace_bytes(2048, 1 << 20, 2048) == 4 * _ws_words(2048, 1 << 20)
    assert tsd.topk_select_workspace_bytes(0, 100, 5) == 0


def test_merge_sharded_rejections():
    m = LIB.topk_merge_sharded
    ok = dict(stride=128, W=4, rows=2, kl=16, k=16)

    def call(**kw):
        a = dict(ok, **kw)
        return m(FAKE, a["stride"], FAKE, FAKE, a["W"], a["rows"], a["kl"],
                 a["k"], FAKE, None, None)
    assert call(W=0) == E["SHAPE"]
    assert call(kl=0) == E["SHAPE"]
    assert call(stride=0) == E["SHAPE"]
    assert call(k=0) == E["K"]
    assert call(k=4097) == E["K"]
    assert call(W=17) == E["UNSUPPORTED"]
    assert call(W=8, kl=4096) == E["UNSUPPORTED"]  # 32,768 candidates
    assert call(W=16, stride=1 << 28) == E["UNSUPPORTED"]  # tokens past 2^31
    assert m(None, 128, FAKE, FAKE, 4, 2, 16, 16, FAKE, None, None) == E["NULL"]
    assert m(None, 128, None, None, 4, 0, 16, 16, None, None, None) == 0


def _append(**kw):
    a = tsd.AppendArgs()
    a.abi_version, a.B, a.page_size, a.max_new = 1, 2, 64, 4
    a.page_table, a.pt_stride, a.num_pages = FAKE, 8, 16
    a.positions, a.n_new = FAKE, FAKE
    a.H_kv, a.D, a.new_dtype, a.kv_dtype = 4, 128, 1, 3
    a.k_new, a.v_new, a.k_pool, a.v_pool = FAKE, FAKE, FAKE, FAKE
    a.k_scale, a.v_scale = FAKE, FAKE
    a.channel_idx, a.label_pool, a.r = FAKE, FAKE, 16
    a.index_dtype, a.index_k_new, a.index_k_pool, a.D_i = 4, FAKE, FAKE, 128
    for k, v in kw.items():
        setattr(a, k, v)
    return LIB.kv_append(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,code", [
    (dict(abi_version=3), "ABI"),
    (dict(page_size=32), "PAGE_SIZE"),
    (dict(B=-1), "SHAPE"),
    (dict(max_new=-1), "SHAPE"),
    (dict(pt_stride=0), "SHAPE"),
    (dict(new_dtype=3), "DTYPE"),
    (dict(kv_dtype=2), "DTYPE"),            # fp16 pool for bf16 rows
    (dict(D=64), "UNSUPPORTED"),
    (dict(H_kv=64), "UNSUPPORTED"),         # H_kv * D > 4096
    (dict(v_new=None), "NULL"),
    (dict(k_scale=None), "NULL"),
    (dict(label_pool=None), "NULL"),
    (dict(r=0), "SHAPE"),
    (dict(r=129), "UNSUPPORTED"),
    (dict(index_dtype=3), "DTYPE"),
    (dict(index_k_pool=None), "NULL"),
    (dict(D_i=64), "UNSUPPORTED"),
    (dict(k_pool=ctypes.c_void_p(0x10004)), "UNSUPPORTED"),  # misaligned
    (dict(page_table=None), "NULL"),
])
def test_append_rejections(kw, code):
    assert _append(**kw) == E[code]


def test_compress_and_expand_rejections():
    assert LIB.tsd_sizeof_compress_args() == ctypes.sizeof(tsd.CompressArgs)

    def comp(**kw):
        a = tsd.CompressArgs()
        a.abi_version, a.B, a.page_size, a.block_size = 1, 2, 64, 4
        a.index_k_pool, a.page_table, a.pt_stride, a.num_pages = FAKE, FAKE, 8, 16
        a.seq_lens, a.from_block, a.max_blocks, a.D_i = FAKE, None, 128, 128
        a.ck_pool, a.cpage_table, a.cpt_stride, a.num_cpages = FAKE, FAKE, 2, 4
        for k, v in kw.items():
            setattr(a, k, v)
        return LIB.index_k_compress(ctypes.byref(a), None)
    assert comp(abi_version=0) == E["ABI"]
    assert comp(page_size=16) == E["PAGE_SIZE"]
    assert comp(block_size=3) == E["UNSUPPORTED"]
    assert comp(block_size=128) == E["UNSUPPORTED"]
    assert comp(D_i=64) == E["UNSUPPORTED"]
    assert comp(cpt_stride=0) == E["SHAPE"]
    assert comp(ck_pool=None) == E["NULL"]
    assert comp(max_blocks=0, ck_pool=None) == 0
    assert comp(ck_pool=0x10008) == E["UNSUPPORTED"]
    assert comp(index_k_pool=0x10004) == E["UNSUPPORTED"]
    x = LIB.expand_blocks
    assert x(FAKE, FAKE, 2, 0, 4, FAKE, 16, FAKE, None, None) == E["K"]
    assert x(FAKE, FAKE, 2, 8, 4, FAKE, 4097, FAKE, None, None) == E["K"]
    assert x(FAKE, FAKE, 2, 8, 5, FAKE, 16, FAKE, None, None) == E["UNSUPPORTED"]
    assert x(None, FAKE, 2, 8, 4, FAKE, 16, FAKE, None, None) == E["NULL"]
    assert x(None, None, 0, 8, 4, None, 16, None, None, None) == 0


def test_append_nothing_to_do():
    assert LIB.kv_append(None, None) == E["NULL"]
    assert _append(B=0, page_table=None, positions=None, n_new=None) == 0
    assert _append(max_new=0) == 0
    # every pool absent: a valid call that stores nothing
    assert _append(k_new=None, channel_idx=None, index_k_new=None) == 0


def _attn(**kw):
    a = AttnArgs()
    a.abi_version, a.B, a.H_q, a.H_kv, a.D = 1, 2, 32, 4, 128
    a.q_dtype, a.q, a.k_pool, a.v_pool = 1, FAKE, FAKE, FAKE
    a.kv_dtype, a.page_size, a.k_scale, a.v_scale = 3, 64, FAKE, FAKE
    a.page_table, a.pt_stride, a.seq_lens, a.num_pages = FAKE, 4, FAKE, 8
    a.idx, a.count, a.H_sel, a.k, a.chunks = FAKE, FAKE, 1, 64, 4
    a.softmax_scale, a.o_part, a.lse_part = 0.088, FAKE, FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return LIB.sparse_gqa_decode(ctypes.byref(a), None)


@pytest.mark.parametrize("kw,code", [
    (dict(abi_version=0), "ABI"),
    (dict(H_q=30), "GQA"),
    (dict(H_sel=2), "GQA"),
    (dict(H_q=68, H_kv=4), "UNSUPPORTED"),
    (dict(D=64), "UNSUPPORTED"),
    (dict(k=0), "K"),
    (dict(chunks=0), "CHUNKS"),
    (dict(chunks=65), "CHUNKS"),
    (dict(kv_dtype=9), "DTYPE"),
    (dict(q_dtype=3), "DTYPE"),
    (dict(kv_dtype=2, q_dtype=1), "DTYPE"),
    (dict(k_scale=None), "NULL"),
    (dict(idx=None), "NULL"),
    (dict(page_size=128), "PAGE_SIZE"),
    (dict(dense_len=-1), "SHAPE"),
    (dict(idx_block=3), "UNSUPPORTED"),
    (dict(idx_block=-1), "UNSUPPORTED"),
    (dict(idx_block=128), "UNSUPPORTED"),
])
def test_attn_rejections(kw, code):
    assert _attn(**kw) == E[code]


def test_attn_empty_batch_and_null():
    assert LIB.sparse_gqa_decode(None, None) == E["NULL"]
    assert _attn(B=0, q=None, idx=None, page_table=None, seq_lens=None) == 0
    assert _attn(B=0, q=None, idx=None, page_table=None, seq_lens=None,
                 idx_block=64) == 0


def test_merge_rejections():
    m = LIB.lse_merge
    assert m(FAKE, FAKE, 4, 0, 128, FAKE, None, None) == E["CHUNKS"]
    assert m(FAKE, FAKE, 4, 65, 128, FAKE, None, None) == E["CHUNKS"]
    assert m(FAKE, FAKE, -1, 4, 128, FAKE, None, None) == E["SHAPE"]
    assert m(FAKE, FAKE, 4, 4, 1024, FAKE, None, None) == E["UNSUPPORTED"]
    assert m(None, FAKE, 4, 4, 128, FAKE, None, None) == E["NULL"]
    assert m(None, None, 0, 4, 128, None, None, None) == 0


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        tsd.lse_merge(torch.zeros(2, 3, 8), torch.zeros(2, 3), torch.zeros(2, 8))


def test_noalloc_rejections():
    """topk_select_noalloc validates like topk_select and refuses a
    selection larger than its built-in scratch before touching the
    device."""
    f = LIB.topk_select_noalloc

    def call(rows=2, max_len=100, k=10, stride=128, scores=FAKE):
        return f(scores, stride, rows, FAKE, max_len, k, FAKE, None, None)
    assert LIB.topk_select_noalloc_max_bytes() == 8 << 20
    assert call(k=0) == E["K"]
    assert call(max_len=200) == E["SHAPE"]
    assert call(rows=-1) == E["SHAPE"]
    assert call(scores=None) == E["NULL"]
    assert call(rows=70000) == E["UNSUPPORTED"]
    assert call(rows=0, scores=None) == 0
    assert call(rows=64, max_len=1 << 20, stride=1 << 20, k=2048) == E["SCRATCH"]
    assert b"scratch" in LIB.tsd_strerror(E["SCRATCH"])
