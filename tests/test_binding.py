"""The Python binding on the host, without a GPU: every wrapper checks the
shapes of its tensors before it checks their placement, so a mis-sized
tensor is rejected with a ValueError before any C call could turn it into an
out-of-bounds device access; and a library built from other sources than
the ones beside it is refused at import."""
import os
import shutil
import subprocess
import sys

import pytest
import torch

import top_sparse_decode_amd as tsd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
I32, F32, U8, BF = torch.int32, torch.float32, torch.uint8, torch.bfloat16


def z(*shape, dtype=I32):
    return torch.zeros(shape, dtype=dtype)


def qsa_kw(**over):
    kw = dict(scores=z(2, 256, dtype=F32), page_table=z(2, 4), seq_lens=z(2),
              num_pages=8, index_q=z(2, 16, 128, dtype=U8),
              index_w=z(2, 16, dtype=F32), index_k_pool=z(512, 128, dtype=U8),
              row_lens_out=z(2))
    kw.update(over)
    return kw


def score(kw):
    kw = dict(kw)
    args = [kw.pop(n) for n in ("scores", "page_table", "seq_lens",
                                "num_pages")]
    tsd.sparse_index_score("qsa", *args, **kw)


def attn_kw(**over):
    kw = dict(q=z(2, 8, 128, dtype=BF), k_pool=z(512, 1, 128, dtype=U8),
              v_pool=z(512, 1, 128, dtype=U8), page_table=z(2, 4),
              seq_lens=z(2), num_pages=8, idx=z(2, 1, 16), count=z(2, 1),
              chunks=4, o_part=z(2, 8, 4, 128, dtype=F32),
              lse_part=z(2, 8, 4, dtype=F32), k_scale=z(8, dtype=F32),
              v_scale=z(8, dtype=F32))
    kw.update(over)
    return kw


def attn(kw):
    kw = dict(kw)
    args = [kw.pop(n) for n in ("q", "k_pool", "v_pool", "page_table",
                                "seq_lens", "num_pages", "idx", "count",
                                "chunks", "o_part", "lse_part")]
    tsd.sparse_gqa_decode(*args, **kw)


@pytest.mark.parametrize("over,what", [
    (dict(scores=z(3, 256, dtype=F32)), "scores"),
    (dict(scores=z(512, dtype=F32)), "scores"),
    (dict(seq_lens=z(3)), "seq_lens"),
    (dict(index_q=z(2, 16, 64, dtype=U8)), "index_k_pool"),
    (dict(index_w=z(2, 15, dtype=F32)), "index_w"),
    (dict(index_k_pool=z(100, 128, dtype=U8)), "slots"),
    (dict(row_lens_out=z(1)), "row_lens_out"),
    (dict(q_pos=z(5)), "q_pos"),
])
def test_score_shapes_rejected(over, what):
    with pytest.raises(ValueError, match=what):
        score(qsa_kw(**over))


def test_score_ds_label_pool_shape():
    kw = dict(scores=z(4, 256, dtype=F32), page_table=z(2, 4), seq_lens=z(2),
              num_pages=8, q=z(2, 8, 128, dtype=BF), channel_idx=z(2, 16),
              label_pool=z(512, 2, 8, dtype=BF))
    with pytest.raises(ValueError, match="label_pool"):
        args = [kw.pop(n) for n in ("scores", "page_table", "seq_lens",
                                    "num_pages")]
        tsd.sparse_index_score("ds", *args, **kw)


def test_well_shaped_host_tensors_reach_the_placement_check():
    with pytest.raises(ValueError, match="CUDA"):
        score(qsa_kw())
    with pytest.raises(ValueError, match="CUDA"):
        attn(attn_kw())


def test_topk_index_shapes_rejected():
    kw = qsa_kw()
    args = [kw.pop(n) for n in ("scores", "page_table", "seq_lens",
                                "num_pages")]
    rl = kw.pop("row_lens_out")
    with pytest.raises(ValueError, match="idx"):
        tsd.sparse_index_topk("qsa", *args, 16, z(2, 15), z(2), z(64, dtype=U8),
                              rl, **kw)
    with pytest.raises(ValueError, match="count"):
        tsd.sparse_index_topk("qsa", *args, 16, z(2, 16), z(3), z(64, dtype=U8),
                              rl, **kw)
    with pytest.raises(ValueError, match="idx"):
        tsd.topk_select(z(2, 256, dtype=F32), z(2), 16, 256, z(2, 8), z(2))
    with pytest.raises(ValueError, match="row_lens"):
        tsd.topk_select(z(2, 256, dtype=F32), z(4), 16, 256, z(2, 16), z(2))


@pytest.mark.parametrize("over,what", [
    (dict(o_part=z(2, 8, 3, 128, dtype=F32)), "o_part"),
    (dict(lse_part=z(2, 8, 5, dtype=F32)), "lse_part"),
    (dict(k_pool=z(100, 1, 128, dtype=U8), v_pool=z(100, 1, 128, dtype=U8)),
     "slots"),
    (dict(v_pool=z(512, 2, 128, dtype=U8)), "v_pool"),
    (dict(k_scale=z(7, dtype=F32)), "k_scale"),
    (dict(idx=z(3, 1, 16)), "idx"),
    (dict(count=z(2, 2)), "count"),
    (dict(q=z(3, 8, 128, dtype=BF)), "q"),
])
def test_attention_shapes_rejected(over, what):
    with pytest.raises(ValueError, match=what):
        attn(attn_kw(**over))


def test_merge_append_blocks_and_sharded_shapes_rejected():
    with pytest.raises(ValueError, match="out"):
        tsd.lse_merge(z(2, 8, 4, 128, dtype=F32), z(2, 8, 4, dtype=F32),
                      z(2, 8, 64, dtype=F32))
    with pytest.raises(ValueError, match="lse_part"):
        tsd.lse_merge(z(2, 8, 4, 128, dtype=F32), z(2, 8, 3, dtype=F32),
                      z(2, 8, 128, dtype=F32))
    with pytest.raises(ValueError, match="k_new"):
        tsd.kv_append(z(2, 4), 8, z(2), z(2), 2, k_new=z(2, 1, 1, 128, dtype=BF),
                      v_new=z(2, 1, 1, 128, dtype=BF),
                      k_pool=z(512, 1, 128, dtype=BF),
                      v_pool=z(512, 1, 128, dtype=BF))
    with pytest.raises(ValueError, match="index_k_pool"):
        tsd.kv_append(z(2, 4), 8, z(2), z(2), 1,
                      index_k_new=z(2, 1, 128, dtype=BF),
                      index_k_pool=z(64, 128, dtype=U8))
    with pytest.raises(ValueError, match="tok"):
        tsd.expand_blocks(z(2, 16), z(2), 4, z(2), z(3, 64))
    with pytest.raises(ValueError, match="idx_local"):
        tsd.topk_merge_sharded(z(4, 2, 256, dtype=F32), z(3, 2, 16), z(4, 2),
                               16, z(2, 16))
    with pytest.raises(ValueError, match="ck_pool"):
        tsd.index_k_compress(z(512, 128, dtype=U8), z(2, 4), 8, z(2),
                             z(10, 128, dtype=U8), z(2, 1), 1, 4, 16)


def test_library_carries_the_digest_of_its_sources():
    from top_sparse_decode_amd import _srchash
    assert tsd._lib.tsd_source_sha256().decode() == _srchash.source_sha256()


def _import_copy(tmp_path, edit):
    """Copy the package (with its built library) and the header to a
    scratch tree, apply ``edit`` to that copy, then import the copy in a
    fresh interpreter. Returns the completed process."""
    dst = tmp_path / "tree"
    shutil.copytree(os.path.join(ROOT, "top_sparse_decode_amd"),
                    dst / "top_sparse_decode_amd",
                    ignore=shutil.ignore_patterns("_build", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "include"), dst / "include")
    edit(dst)
    env = dict(os.environ, PYTHONPATH=str(dst))
    env.pop("TSD_LIB", None)
    return subprocess.run([sys.executable, "-c", "import top_sparse_decode_amd"],
                          cwd=str(dst), env=env, capture_output=True, text=True,
                          timeout=300)


def test_unchanged_copy_imports(tmp_path):
    r = _import_copy(tmp_path, lambda d: None)
    assert r.returncode == 0, r.stderr


def test_changed_source_refuses_the_stale_library(tmp_path):
    def edit(d):
        src = d / "top_sparse_decode_amd" / "csrc" / "lse_merge.hip"
        src.write_text(src.read_text() + "\n// changed\n")
    r = _import_copy(tmp_path, edit)
    assert r.returncode != 0
    assert "built from other sources" in r.stderr
