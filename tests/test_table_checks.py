"""The host-side table checks of the binding (CPU): valid tables from the input
generators pass, and each kind of entry a kernel would read out of range is
refused with ValueError."""
import pytest
import torch

import gqa_attention_forward_attn_amd as gqa
import workloads as W


def dec_inputs():
    return W.make_decode(3, 8, 2, 64, "bf16", seed=5, len_lo=1, len_hi=300, page_size=16)


def test_decode_tables_valid():
    inp = dec_inputs()
    gqa.check_decode_tables(inp.seq_lens, inp.block_table, 16, inp.k_cache.shape[0], inp.max_kv_len)
    gqa.check_decode_tables(inp.seq_lens, None, 0, 0, inp.max_kv_len)


@pytest.mark.parametrize("bad", ["negative_len", "long_len", "page_high", "page_negative", "row_short"])
def test_decode_tables_refused(bad):
    inp = dec_inputs()
    lens, bt = inp.seq_lens.clone(), inp.block_table.clone()
    n_pages, max_kv = inp.k_cache.shape[0], inp.max_kv_len
    if bad == "negative_len":
        lens[1] = -1
    elif bad == "long_len":
        lens[0] = max_kv + 1
    elif bad == "page_high":
        bt[2, 0] = n_pages
    elif bad == "page_negative":
        bt[0, (int(lens[0]) - 1) // 16] = -1   # the last page the sequence uses
    elif bad == "row_short":
        bt = bt[:, :1].contiguous()
        lens[0] = 17                            # needs two pages
        max_kv = 10 ** 6
    with pytest.raises(ValueError):
        gqa.check_decode_tables(lens, bt, 16, n_pages, max_kv)


def pf_inputs():
    return W.make_paged_prefill(4, 8, 2, 64, "bf16", seed=6, q_lo=1, q_hi=40, prefix_lo=0, prefix_hi=60,
                                page_size=8)


def pf_check(inp, qo=None, kvp=None, idx=None, last="same", max_q=None):
    gqa.check_paged_prefill_tables(inp.qo_indptr if qo is None else qo, inp.kv_indptr if kvp is None else kvp,
                                   inp.kv_indices if idx is None else idx,
                                   inp.kv_last_page_len if isinstance(last, str) else last,
                                   inp.k_cache.shape[0], 8, inp.max_q_len if max_q is None else max_q,
                                   inp.q.shape[0])


def test_paged_prefill_tables_valid():
    inp = pf_inputs()
    pf_check(inp)
    pf_check(inp, last=None)


@pytest.mark.parametrize("bad", ["qo_start", "qo_decreasing", "qo_past_q", "too_many_queries", "page_high",
                                 "page_negative", "last_zero", "last_long", "kv_past_indices"])
def test_paged_prefill_tables_refused(bad):
    inp = pf_inputs()
    qo, kvp, idx, last = (inp.qo_indptr.clone(), inp.kv_indptr.clone(), inp.kv_indices.clone(),
                          inp.kv_last_page_len.clone())
    max_q = None
    if bad == "qo_start":
        qo[0] = 1
    elif bad == "qo_decreasing":
        qo[2] = qo[1] - 1
    elif bad == "qo_past_q":
        qo[-1] = inp.q.shape[0] + 1
    elif bad == "too_many_queries":
        max_q = int((qo[1:] - qo[:-1]).max()) - 1
    elif bad == "page_high":
        idx[0] = inp.k_cache.shape[0]
    elif bad == "page_negative":
        idx[-1] = -1
    elif bad == "last_zero":
        last[0] = 0
    elif bad == "last_long":
        last[1] = 9
    elif bad == "kv_past_indices":
        kvp[-1] = idx.numel() + 1
    with pytest.raises(ValueError):
        pf_check(inp, qo, kvp, idx, last, max_q)
