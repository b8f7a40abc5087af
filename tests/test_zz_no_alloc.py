"""The allocation-free decode entry point (attn_decode_splitk_noalloc: the
library's fixed device scratch instead of a caller workspace) against the
entry point it extends (attn_decode_splitk with a workspace), through the C
ABI, on two calls in a row, the second one smaller; both also against the
oracle."""
import numpy as np
import pytest
import torch

import oracle
import gqa_attention_forward_attn_amd as gqa
import workloads as W

pytestmark = pytest.mark.gpu

TOL_O, TOL_L = 2e-2, 1e-3


def _run_both(inp, n_splits, scale):
    q, kc, vc = inp.q.cuda(), inp.k_cache.cuda(), inp.v_cache.cuda()
    sl, bt = inp.seq_lens.cuda(), inp.block_table.cuda()
    o_ws = torch.full_like(q, float("nan"))
    l_ws = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    gqa.attn_decode_splitk(q, kc, vc, sl, block_table=bt, n_splits=n_splits, scale=scale,
                           max_kv_len=inp.max_kv_len, out=o_ws, lse=l_ws)
    o_na = torch.full_like(q, float("nan"))
    l_na = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    gqa.attn_decode_splitk_noalloc(q, kc, vc, sl, o_na, l_na, block_table=bt, n_splits=n_splits, scale=scale,
                                   max_kv_len=inp.max_kv_len)
    torch.cuda.synchronize()
    return o_ws.cpu(), l_ws.cpu(), o_na.cpu(), l_na.cpu()


def _check_oracle(inp, scale, o, l):
    o_ref, l_ref = oracle.attn_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, scale,
                                      block_table=inp.block_table, max_kv_len=inp.max_kv_len)
    o, l = o.double().numpy(), l.double().numpy()
    assert not np.isnan(o).any() and not np.isnan(l).any()
    assert np.array_equal(np.isneginf(l), np.isneginf(l_ref))
    fin = ~np.isneginf(l_ref)
    assert np.abs(o - o_ref).max() <= TOL_O
    assert np.abs(l[fin] - l_ref[fin]).max() <= TOL_L


def test_noalloc_equals_workspace_call_twice_second_smaller():
    # first call: the paged decode workload's shape (16 sequences, 32 heads, 16 splits)
    print("no-alloc decode: paged decode workload", flush=True)
    spec = W.PAGED_DECODE
    inp = W.make_decode_spec(spec)
    scale = W.fp32_scale(spec.D)
    o_ws, l_ws, o_na, l_na = _run_both(inp, spec.n_splits, scale)
    assert torch.equal(o_ws, o_na) and torch.equal(l_ws, l_na)
    _check_oracle(inp, scale, o_na, l_na)
    # second call, smaller (3 sequences, 8 heads, D = 64, 5 splits, an empty
    # sequence): the scratch still holds the first call's partials
    print("no-alloc decode: small second call", flush=True)
    inp2 = W.make_decode(3, 8, 2, 64, "f16", seed=77, len_lo=0, len_hi=700, page_size=16)
    inp2.seq_lens[1] = 0
    o_ws, l_ws, o_na, l_na = _run_both(inp2, 5, 0.125)
    assert torch.equal(o_ws, o_na) and torch.equal(l_ws, l_na)
    _check_oracle(inp2, 0.125, o_na, l_na)


def test_noalloc_rejects_requests_beyond_the_scratch():
    L = gqa.lib()
    p = [None] * 7
    # 1024 x 32 x 16 chunks x (128 + 1) x 4 bytes = 270 MB > 32 MiB
    rc = L.attn_decode_splitk_noalloc(*p, 4, 256, 1024, 32, 8, 128, 4096, 0.088, 16, gqa.GQA_BF16, None)
    assert rc == 3  # GQA_ERR_WORKSPACE
