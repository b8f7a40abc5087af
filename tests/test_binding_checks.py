"""The Python binding refuses tensors the kernels would read or write out of
bounds, before any launch (CPU only: these calls never reach the library).

Shapes are checked before devices, so host tensors exercise every shape rule;
a call whose shapes are right but whose tensors are on the host is refused too.
"""
import pytest
import torch

import gqa_attention_forward_attn_amd as gqa

bf = torch.bfloat16


def _prefill(B=1, Hq=4, Hkv=2, Lq=8, Lk=8, D=64, dtype=bf):
    return (torch.zeros(B, Hq, Lq, D, dtype=dtype), torch.zeros(B, Hkv, Lk, D, dtype=dtype),
            torch.zeros(B, Hkv, Lk, D, dtype=dtype))


def test_fwd_shape_mismatches():
    q, k, v = _prefill()
    with pytest.raises(ValueError):
        gqa.attn_fwd(q, k[..., :32], v[..., :32])          # head dims differ
    with pytest.raises(ValueError):
        gqa.attn_fwd(q, k, v[:, :, :4])                    # v shorter than k
    with pytest.raises(ValueError):
        gqa.attn_fwd(q, k, v[:, :1])                       # v heads differ
    with pytest.raises(ValueError):
        gqa.attn_fwd(q[0], k, v)                           # 3-D q
    with pytest.raises(TypeError):
        gqa.attn_fwd(q, k.float(), v)                      # dtype mix
    with pytest.raises(ValueError):
        gqa.attn_fwd(q, k, v, kernel="fastest")            # unknown kernel name


def test_fwd_host_tensors_refused():
    q, k, v = _prefill()
    with pytest.raises(ValueError, match="GPU"):
        gqa.attn_fwd(q, k, v)


def test_paged_prefill_shape_mismatches():
    q = torch.zeros(10, 4, 64, dtype=bf)
    pool = torch.zeros(6, 16, 2, 64, dtype=bf)
    qo = torch.tensor([0, 4, 10], dtype=torch.int32)
    kvp = torch.tensor([0, 2, 5], dtype=torch.int32)
    idx = torch.arange(5, dtype=torch.int32)
    with pytest.raises(ValueError):
        gqa.attn_prefill_paged(q, pool[..., :32], pool, qo, kvp, idx, 6)
    with pytest.raises(ValueError):
        gqa.attn_prefill_paged(q, pool, pool, qo, kvp[:2], idx, 6)          # kv_indptr too short
    with pytest.raises(ValueError):
        gqa.attn_prefill_paged(q, pool, pool, qo, kvp, idx, 6,
                               kv_last_page_len=torch.ones(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU"):
        gqa.attn_prefill_paged(q, pool, pool, qo, kvp, idx, 6)


def _decode(B=3, Hq=8, Hkv=2, D=64, pages=12, ps=16, max_pages=4):
    q = torch.zeros(B, Hq, D, dtype=bf)
    pool = torch.zeros(pages, ps, Hkv, D, dtype=bf)
    lens = torch.full((B,), 20, dtype=torch.int32)
    bt = torch.zeros(B, max_pages, dtype=torch.int32)
    return q, pool, lens, bt


def test_decode_shape_mismatches():
    q, pool, lens, bt = _decode()
    with pytest.raises(ValueError):
        gqa.attn_decode_splitk(q, pool[..., :32], pool[..., :32], lens, block_table=bt)   # D differs
    with pytest.raises(ValueError):
        gqa.attn_decode_splitk(q, pool, pool[:6], lens, block_table=bt)                   # v differs
    with pytest.raises(ValueError):
        gqa.attn_decode_splitk(q, pool, pool, lens[:2], block_table=bt)                   # seq_lens != B
    with pytest.raises(ValueError):
        gqa.attn_decode_splitk(q, pool, pool, lens, block_table=bt[:2])                   # table rows != B
    with pytest.raises(ValueError):
        gqa.attn_decode_splitk(q, pool, pool, lens, block_table=bt, max_kv_len=4 * 16 + 1)  # past the table
    with pytest.raises(TypeError):
        gqa.attn_decode_splitk(q.float(), pool, pool, lens, block_table=bt)
    with pytest.raises(ValueError, match="GPU"):
        gqa.attn_decode_splitk(q, pool, pool, lens, block_table=bt)


def test_decode_dense_row_stride_must_match():
    q = torch.zeros(2, 8, 64, dtype=bf)
    k = torch.zeros(2, 2, 100, 64, dtype=bf)
    lens = torch.tensor([50, 100], dtype=torch.int32)
    # the dense row stride is k.shape[2]; any other max_kv_len would misread k/v
    for bad in (99, 101):
        with pytest.raises(ValueError, match="row stride"):
            gqa.attn_decode_splitk(q, k, k, lens, max_kv_len=bad)
    with pytest.raises(ValueError):
        gqa.attn_decode_splitk(q, k[:1], k[:1], lens)                                    # B differs
    with pytest.raises(ValueError, match="GPU"):
        gqa.attn_decode_splitk(q, k, k, lens, max_kv_len=100)


def test_decode_multi_and_fp8_shapes():
    q, pool, lens, bt = _decode()
    with pytest.raises(ValueError):
        gqa.attn_decode_splitk_multi(q, pool, pool, lens, block_table=bt)                 # 3-D q
    q4 = q.unsqueeze(2).repeat(1, 1, 3, 1)
    with pytest.raises(ValueError, match="GPU"):
        gqa.attn_decode_splitk_multi(q4, pool, pool, lens, block_table=bt)
    k8 = torch.zeros(12, 16, 2, 64, dtype=torch.uint8)
    ss = torch.zeros(12, 16, 2, dtype=torch.int32)
    with pytest.raises(TypeError):
        gqa.attn_decode_splitk_fp8(q, pool, pool, ss, ss, lens, block_table=bt)          # not E4M3 bytes
    with pytest.raises(ValueError):
        gqa.attn_decode_splitk_fp8(q, k8, k8, ss[:, :8], ss, lens, block_table=bt)       # scale-shift shape
    with pytest.raises(ValueError, match="GPU"):
        gqa.attn_decode_splitk_fp8(q, k8, k8, ss, ss, lens, block_table=bt)
