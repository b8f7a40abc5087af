"""Host-side arithmetic of bench.py, on the CPU: the algorithmic flop and byte
counts that the reported throughputs and roofline fractions divide by, checked
against independent counts over the generated inputs; the traffic figure; and
the one-GPU refusal."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def mask_count(q_len, kv_len, causal):
    """Visible (query, key) pairs by materialising the bottom-right mask."""
    i = np.arange(q_len)[:, None]
    j = np.arange(kv_len)[None, :]
    vis = np.ones((q_len, kv_len), dtype=bool) if not causal else (j <= i + (kv_len - q_len))
    return int(vis.sum())


@pytest.mark.parametrize("q_len,kv_len", [(1, 1), (5, 5), (7, 20), (20, 7), (64, 64), (0, 9), (9, 0),
                                          (130, 333), (1024, 4096)])
@pytest.mark.parametrize("causal", [True, False])
def test_visible_pairs_equals_mask_count(q_len, kv_len, causal):
    assert bench.visible_pairs(q_len, kv_len, causal) == mask_count(q_len, kv_len, causal)


def test_prefill_flops_of_the_workloads():
    # 4 D flops per visible pair (2 D for the score, 2 D for P.V), every query head
    assert bench.prefill_flops(W.CAUSAL_GQA_PREFILL) == 4 * 128 * 2 * 32 * (2048 * 2049 // 2) == 68_753_031_168
    assert bench.prefill_flops(W.CAUSAL_GQA_OFFSET) == 4 * 128 * 32 * mask_count(1024, 4096, True) == 60_137_930_752
    assert bench.prefill_flops(W.MHA_NONCAUSAL_FP16) == 4 * 64 * 4 * 16 * 4096 * 4096
    assert bench.prefill_flops(W.CAUSAL_GQA_FP32) == 4 * 64 * 4 * (128 * 129 // 2)


@pytest.mark.parametrize("q_len,fp8", [(1, False), (3, False), (1, True)])
def test_decode_bytes_equal_the_bytes_of_the_gathered_rows(q_len, fp8):
    spec = W.DecodeSpec("small", 3, 8, 2, 64, "bf16", 1, 700, 64, 16, 4, 99, q_len)
    if fp8:
        inp = W.make_decode_fp8_spec(spec)
        k, v, extra = inp.k8, inp.v8, (inp.k_ss, inp.v_ss)
    else:
        inp = W.make_decode_spec(spec)
        k, v, extra = inp.k_cache, inp.v_cache, ()
    # the K/V rows (and scale-shift words) each sequence's tokens occupy, gathered page by page
    kv = 0
    pages = 0
    for b in range(spec.B):
        n = int(inp.seq_lens[b])
        ids = inp.block_table[b, :(n + spec.page_size - 1) // spec.page_size].long()
        pages += len(ids)
        for t in (k, v) + extra:
            kv += t[ids].reshape(-1, *t.shape[2:])[:n].numel() * t.element_size()
    q = inp.q
    o_bytes = q.numel() * q.element_size()
    lse_bytes = q.numel() // spec.D * 4
    meta = pages * 4 + spec.B * 4  # page ids read + sequence lengths
    assert bench.decode_bytes(spec, inp, fp8=fp8) == kv + 2 * o_bytes + lse_bytes + meta


def test_workload_decode_bytes():
    # the figure the decode profiles quote for the paged decode workload
    inp = W.make_decode_spec(W.PAGED_DECODE)
    assert bench.decode_bytes(W.PAGED_DECODE, inp) == 1_049_872_388


def test_traffic_matches_the_recorded_source_only(tmp_path, monkeypatch):
    # the recorded counters count for the source they were taken on (by sha1),
    # scaled by the copy calibration; any other source reports no traffic
    import hashlib
    m = dict(bench.TRAFFIC_MEASUREMENT)
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel source the counters were taken on")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.TRAFFIC_MEASUREMENT, "source", "k.hip")
    monkeypatch.setitem(bench.TRAFFIC_MEASUREMENT, "sha1", hashlib.sha1(src.read_bytes()).hexdigest())
    copy_kib = bench.COPY_BYTES / 1024
    want = m["fetch_kib"] * 1024 * copy_kib / m["copy_fetch_kib"] + m["write_kib"] * 1024 * copy_kib / m["copy_write_kib"]
    assert bench.measured_traffic() == int(round(want))
    src.write_bytes(b"changed")
    assert bench.measured_traffic() is None


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout
