"""topk_select_noalloc (the workspace in the library's fixed device scratch,
nothing allocated) against topk_select with a caller workspace, both called
through the C ABI on the same scores: two calls in a row on the chunked
selection path, the second with a smaller input, a third on the
one-workgroup path, each bit-identical to topk_select; then a selection too
large for the scratch is rejected with nothing written."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import top_sparse_decode_amd as tsd

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
E_SCRATCH = -12


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _case(rows, stride, lens, levels, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    # few distinct levels: many ties at every threshold
    s = torch.randint(0, levels, (rows, stride), generator=g, device=DEV)
    s = (s.float() - levels / 2) / 7.0
    return s.contiguous(), torch.tensor(lens, dtype=torch.int32, device=DEV)


def _select_both(s, lens, k, max_len):
    rows, stride = s.shape
    lib = tsd._lib
    idx_a = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    cnt_a = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    idx_b, cnt_b = idx_a.clone(), cnt_a.clone()
    nbytes = tsd.topk_select_workspace_bytes(rows, max_len, k)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    rc = lib.topk_select(_p(s), stride, rows, _p(lens), max_len, k, _p(idx_a),
                         _p(cnt_a), _p(ws), nbytes, _stream())
    assert rc == 0, rc
    rc = lib.topk_select_noalloc(_p(s), stride, rows, _p(lens), max_len, k,
                                 _p(idx_b), _p(cnt_b), _stream())
    assert rc == 0, rc
    torch.cuda.synchronize()
    assert torch.equal(idx_a, idx_b)
    assert torch.equal(cnt_a, cnt_b)
    return idx_b.cpu().numpy(), cnt_b.cpu().numpy()


def test_noalloc_matches_topk_select_on_consecutive_calls():
    assert tsd._lib.topk_select_noalloc_max_bytes() == 8 << 20
    # call 1: 8 rows of up to 262,144 entries, k = 2048 (2.3 MB of scratch)
    lens1 = [262144, 262144, 200001, 131072, 4097, 65536, 0, 262143]
    s1, l1 = _case(8, 262144, lens1, 50, seed=1)
    print("noalloc call 1: rows 8 stride 262144 k 2048", flush=True)
    idx1, cnt1 = _select_both(s1, l1, 2048, 262144)
    ref_idx, ref_cnt = oracle.topk(s1[[0, 4, 6]].cpu().numpy(),
                                   np.array(lens1)[[0, 4, 6]], 2048)
    np.testing.assert_array_equal(idx1[[0, 4, 6]], ref_idx)
    np.testing.assert_array_equal(cnt1[[0, 4, 6]], ref_cnt)
    # call 2: smaller (3 rows of up to 70,000, k = 300), same scratch
    lens2 = [70000, 33000, 69999]
    s2, l2 = _case(3, 70000, lens2, 1000, seed=2)
    print("noalloc call 2: rows 3 stride 70000 k 300", flush=True)
    idx2, cnt2 = _select_both(s2, l2, 300, 70000)
    ref_idx, ref_cnt = oracle.topk(s2.cpu().numpy(), np.array(lens2), 300)
    np.testing.assert_array_equal(idx2, ref_idx)
    np.testing.assert_array_equal(cnt2, ref_cnt)
    # call 3: rows short enough for the one-workgroup selection
    lens3 = [5000, 17]
    s3, l3 = _case(2, 5000, lens3, 30, seed=3)
    print("noalloc call 3: rows 2 stride 5000 k 64", flush=True)
    _select_both(s3, l3, 64, 5000)


def test_noalloc_rejects_selections_beyond_its_scratch():
    rows, stride, k = 64, 1 << 20, 2048
    assert tsd.topk_select_workspace_bytes(rows, stride, k) > 8 << 20
    s = torch.zeros((rows, stride), device=DEV)  # rejected before any read
    lens = torch.zeros(rows, dtype=torch.int32, device=DEV)
    idx = torch.full((rows, k), -7, dtype=torch.int32, device=DEV)
    rc = tsd._lib.topk_select_noalloc(_p(s), stride, rows, _p(lens), stride,
                                      k, _p(idx), None, _stream())
    torch.cuda.synchronize()
    assert rc == E_SCRATCH
    assert b"scratch" in tsd._lib.tsd_strerror(rc)
    assert bool((idx == -7).all())
