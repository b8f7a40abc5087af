"""Benchmark: GQA attention forward on one MI355X.

Prints ONE JSON line.  The headline workload is causal GQA prefill in bf16
(B=2, Hq=32, Hkv=8, S=2048, D=128): one step is one attn_fwd call over that
batch, inputs already resident in HBM.  `value` is TFLOP/s counted on the
visible (query, key) pairs only (4*D flop per pair; masked work is not
credited).  The other workloads (fp32 correctness shape, bottom-right offset
prefill, non-causal fp16 MHA, split-K paged decode over a 16-bit and over an
E4M3 cache, decode with four queries per sequence, ragged prefill over a paged
cache, the headline prefill and the paged decode with an additive bias, the
backward of the split-K merge) are timed the same way and reported under
"workloads".

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--only NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gqa_attention_forward_attn_amd as gqa  # noqa: E402
import workloads as W  # noqa: E402

PEAK_MFMA_16BIT_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA (2.5 PFLOP/s published)
PEAK_MFMA_F32_TFLOPS = 157.3      # MI355X fp32 MFMA
PEAK_HBM_GBPS = 8000.0            # MI355X HBM3E

PRIMARY = W.CAUSAL_GQA_PREFILL
METRIC = "attention fwd TFLOP/s + % bf16 MFMA peak; decode GB/s + % HBM peak"

# HBM traffic per launch of the dominant kernel: rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch, one pass each, profiles/prefill_fwd_pp_causal_gqa_prefill.md),
# scaled by what the same counters read for `--only hbm_copy` (COPY_BYTES read
# and written).  The figures hold for the kernel source they were taken on; any
# other source reports traffic null.
TRAFFIC_MEASUREMENT = {
    "source": "gqa_attention_forward_attn_amd/csrc/prefill_pp.hip",
    "sha1": "148b57d01e21ee7c10f1392df0cb649002db4a05",
    "fetch_kib": 24780.1, "write_kib": 33280.0,
    "copy_fetch_kib": 262155.5, "copy_write_kib": 524288.0,
}


def measured_traffic():
    m = TRAFFIC_MEASUREMENT
    try:
        with open(os.path.join(ROOT, m["source"]), "rb") as f:
            if hashlib.sha1(f.read()).hexdigest() != m["sha1"]:
                return None
    except OSError:
        return None
    copy_kib = COPY_BYTES / 1024
    fetch = m["fetch_kib"] * 1024 * copy_kib / m["copy_fetch_kib"]
    write = m["write_kib"] * 1024 * copy_kib / m["copy_write_kib"]
    return int(round(fetch + write))


def visible_pairs(q_len: int, kv_len: int, causal: bool) -> int:
    if not causal:
        return q_len * kv_len
    delta = kv_len - q_len
    return int(sum(max(0, min(kv_len, i + 1 + delta)) for i in range(q_len)))


def prefill_flops(spec) -> int:
    return 4 * spec.D * spec.B * spec.Hq * visible_pairs(spec.q_len, spec.kv_len, spec.causal)


def decode_bytes(spec, inp, fp8=False) -> int:
    elt = 2
    tokens = int(inp.seq_lens.to(torch.int64).sum())
    pages = int(sum((int(s) + spec.page_size - 1) // spec.page_size for s in inp.seq_lens))
    # K and V: 16-bit elements, or E4M3 bytes plus one 4-byte scale-shift word per token row and head
    kv = 2 * tokens * spec.Hkv * (spec.D + 4 if fp8 else spec.D * elt)
    qo = 2 * spec.B * spec.Hq * spec.q_len * spec.D * elt
    lse = spec.B * spec.Hq * spec.q_len * 4
    meta = 4 * pages + 4 * spec.B
    return kv + qo + lse + meta


def time_launches(fn, steps: int, warmup: int):
    """Warm up, then time `steps` back-to-back calls: wall time around the loop
    (synchronize on both sides) and one HIP event pair around it on the stream
    the library launches on (torch's current stream), whose span / steps is the
    mean launch duration (`kernel_ms_mean`).  A second pass records an event
    pair around every single call: those spans (`call_span_ms_min`,
    `call_span_ms_p90`) also hold each call's own dispatch gap, so they are
    longer than the back-to-back mean and describe the spread only."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = start.elapsed_time(end) * 1e-3 / steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)]) * 1e-3
    return wall, mean, per


def bench_prefill(spec, steps, warmup):
    q, k, v = W.make_prefill_spec(spec)
    dev = torch.device("cuda:0")
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    scale = W.fp32_scale(spec.D)

    def step():
        gqa.attn_fwd(q, k, v, causal=spec.causal, scale=scale, out=o, lse=lse)

    wall, kern_s, per = time_launches(step, steps, warmup)
    flops = prefill_flops(spec)
    peak = PEAK_MFMA_F32_TFLOPS if spec.dtype == "f32" else PEAK_MFMA_16BIT_TFLOPS
    return {
        "workload": spec.name, "dtype": spec.dtype, "causal": spec.causal,
        "shape": {"B": spec.B, "Hq": spec.Hq, "Hkv": spec.Hkv, "q_len": spec.q_len,
                  "kv_len": spec.kv_len, "D": spec.D},
        "flop_per_launch": flops,
        "ms_per_step": wall / steps * 1e3,
        "kernel_ms_mean": kern_s * 1e3, "call_span_ms_min": float(per.min()) * 1e3,
        "call_span_ms_p90": float(np.percentile(per, 90)) * 1e3,
        "tflops": flops * steps / wall / 1e12,
        "kernel_tflops": flops / kern_s / 1e12,
        "peak_tflops": peak,
        "frac_of_peak": flops / kern_s / 1e12 / peak,
    }


COPY_BYTES = 512 << 20


def bench_decode_fp8(spec, steps, warmup):
    inp = W.make_decode_fp8_spec(spec)
    dev = torch.device("cuda:0")
    q = inp.q.to(dev)
    k8, v8, kss, vss = (t.to(dev) for t in (inp.k8, inp.v8, inp.k_ss, inp.v_ss))
    sl, bt = inp.seq_lens.to(dev), inp.block_table.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    ws = torch.empty(gqa.decode_workspace_bytes(spec.B, spec.Hq, spec.D, spec.n_splits), dtype=torch.uint8,
                     device=dev)
    scale = W.fp32_scale(spec.D)

    def step():
        gqa.attn_decode_splitk_fp8(q, k8, v8, kss, vss, sl, block_table=bt, n_splits=spec.n_splits, scale=scale,
                                   max_kv_len=inp.max_kv_len, workspace=ws, out=o, lse=lse)

    wall, kern_s, per = time_launches(step, steps, warmup)
    nbytes = decode_bytes(spec, inp, fp8=True)
    tokens = int(inp.seq_lens.to(torch.int64).sum())
    return {
        "workload": spec.name, "dtype": "e4m3 K/V, " + spec.dtype + " q/o",
        "shape": {"B": spec.B, "Hq": spec.Hq, "Hkv": spec.Hkv, "D": spec.D, "page_size": spec.page_size,
                  "n_splits": spec.n_splits, "sum_kv_len": tokens},
        "bytes_per_step": nbytes,
        "workspace_bytes_rw": 2 * spec.B * spec.Hq * spec.n_splits * (spec.D + 1) * 4,
        "ms_per_step": wall / steps * 1e3,
        "kernel_ms_mean": kern_s * 1e3, "call_span_ms_min": float(per.min()) * 1e3,
        "gbps": nbytes * steps / wall / 1e9,
        "kernel_gbps": nbytes / kern_s / 1e9,
        "tokens_per_s": tokens / kern_s,
        "peak_gbps": PEAK_HBM_GBPS,
        "frac_of_peak": nbytes / kern_s / 1e9 / PEAK_HBM_GBPS,
    }


def bench_prefill_bias(spec, steps, warmup):
    """attn_fwd_bias on the headline shape with a per-head bias [1, Hq, q_len,
    kv_len] (the four-wave kernel's bias form)."""
    q, k, v, bias = W.make_prefill_bias_spec(spec)
    dev = torch.device("cuda:0")
    q, k, v, bias = q.to(dev), k.to(dev), v.to(dev), bias.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    scale = W.fp32_scale(spec.D)

    def step():
        gqa.attn_fwd_bias(q, k, v, bias, causal=spec.causal, scale=scale, out=o, lse=lse)

    wall, kern_s, per = time_launches(step, steps, warmup)
    flops = prefill_flops(spec)
    return {
        "workload": spec.name, "dtype": spec.dtype, "causal": spec.causal,
        "shape": {"B": spec.B, "Hq": spec.Hq, "Hkv": spec.Hkv, "q_len": spec.q_len,
                  "kv_len": spec.kv_len, "D": spec.D, "bias": [1, spec.Hq, spec.q_len, spec.kv_len]},
        "kernel": "prefill_fwd_pp<bf16, D=128, causal, NH=4, bias>",
        "flop_per_launch": flops,
        "bias_bytes": bias.numel() * bias.element_size(),
        "ms_per_step": wall / steps * 1e3,
        "kernel_ms_mean": kern_s * 1e3, "call_span_ms_min": float(per.min()) * 1e3,
        "tflops": flops * steps / wall / 1e12,
        "kernel_tflops": flops / kern_s / 1e12,
        "peak_tflops": PEAK_MFMA_16BIT_TFLOPS,
        "frac_of_peak": flops / kern_s / 1e12 / PEAK_MFMA_16BIT_TFLOPS,
    }


def decode_bias_bytes(spec, inp) -> int:
    """Bias bytes a decode step needs: one 16-bit value per (sequence, head,
    query, key)."""
    return int(inp.seq_lens.to(torch.int64).sum()) * spec.Hq * spec.q_len * 2


def bench_decode_bias(spec, steps, warmup):
    """attn_decode_splitk_bias on the paged decode shape with a bias per
    (sequence, head) over its keys."""
    inp, bias = W.make_decode_bias_spec(spec)
    dev = torch.device("cuda:0")
    q = inp.q.to(dev).reshape(spec.B, spec.Hq, spec.q_len, spec.D)
    kc, vc = inp.k_cache.to(dev), inp.v_cache.to(dev)
    sl, bt, bias = inp.seq_lens.to(dev), inp.block_table.to(dev), bias.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    ws = torch.empty(gqa.decode_workspace_bytes_multi(spec.B, spec.Hq, spec.q_len, spec.D, spec.n_splits),
                     dtype=torch.uint8, device=dev)
    scale = W.fp32_scale(spec.D)

    def step():
        gqa.attn_decode_splitk_bias(q, kc, vc, sl, bias, block_table=bt, n_splits=spec.n_splits, scale=scale,
                                    max_kv_len=inp.max_kv_len, workspace=ws, out=o, lse=lse)

    wall, kern_s, per = time_launches(step, steps, warmup)
    nbytes = decode_bytes(spec, inp) + decode_bias_bytes(spec, inp)
    return {
        "workload": spec.name, "dtype": spec.dtype,
        "shape": {"B": spec.B, "Hq": spec.Hq, "Hkv": spec.Hkv, "D": spec.D, "q_len": spec.q_len,
                  "page_size": spec.page_size, "n_splits": spec.n_splits,
                  "sum_kv_len": int(inp.seq_lens.to(torch.int64).sum()),
                  "bias": [spec.B, spec.Hq, spec.q_len, inp.max_kv_len]},
        "bytes_per_step": nbytes,
        "bias_bytes": decode_bias_bytes(spec, inp),
        "ms_per_step": wall / steps * 1e3,
        "kernel_ms_mean": kern_s * 1e3, "call_span_ms_min": float(per.min()) * 1e3,
        "gbps": nbytes * steps / wall / 1e9,
        "kernel_gbps": nbytes / kern_s / 1e9,
        "peak_gbps": PEAK_HBM_GBPS,
        "frac_of_peak": nbytes / kern_s / 1e9 / PEAK_HBM_GBPS,
    }


def merge_backward_bytes(spec) -> int:
    """Bytes of one merge backward: read o_parts, lse_parts, o, lse, d_o, d_lse;
    write d_o_parts and d_lse_parts (fp32)."""
    S, D = spec.n_splits, spec.D
    return spec.rows * 4 * (2 * S * D + 2 * S + 2 * D + 2)


def bench_merge_backward(spec, steps, warmup):
    """attn_splitk_merge_backward over the partials of a split-KV prefill.  The
    merged (o, lse) it takes are formed from the partials with torch before the
    timed region (inputs of the backward, not part of what is timed)."""
    dev = torch.device("cuda:0")
    op, lp, d_o, d_lse = (t.to(dev) for t in W.make_merge_backward_spec(spec))
    lse = torch.logsumexp(lp.double(), dim=-1)
    w = torch.where(torch.isfinite(lse)[:, None], torch.exp(lp.double() - lse[:, None]), torch.zeros_like(lp.double()))
    o = (w[..., None] * op.double()).sum(dim=-2).float()
    lse = lse.float()
    dop = torch.empty_like(op)
    dlp = torch.empty_like(lp)

    def step():
        gqa.attn_splitk_merge_backward(op, lp, o, lse, d_o, d_lse, d_o_parts=dop, d_lse_parts=dlp)

    wall, kern_s, per = time_launches(step, steps, warmup)
    nbytes = merge_backward_bytes(spec)
    return {
        "workload": spec.name, "dtype": "f32",
        "shape": {"rows": spec.rows, "n_splits": spec.n_splits, "D": spec.D},
        "kernel": "merge_backward_vec_kernel<32, 1, 2> (one wave per row, two partials at a time, 16-byte accesses)",
        "bytes_per_step": nbytes,
        "ms_per_step": wall / steps * 1e3,
        "kernel_ms_mean": kern_s * 1e3, "call_span_ms_min": float(per.min()) * 1e3,
        "gbps": nbytes * steps / wall / 1e9,
        "kernel_gbps": nbytes / kern_s / 1e9,
        "peak_gbps": PEAK_HBM_GBPS,
        "frac_of_peak": nbytes / kern_s / 1e9 / PEAK_HBM_GBPS,
    }


def bench_paged_prefill(spec, steps, warmup):
    inp = W.make_paged_prefill_spec(spec)
    dev = torch.device("cuda:0")
    q = inp.q.to(dev)
    kc, vc = inp.k_cache.to(dev), inp.v_cache.to(dev)
    qo, kvp, idx, last = (t.to(dev) for t in (inp.qo_indptr, inp.kv_indptr, inp.kv_indices,
                                                 inp.kv_last_page_len))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    scale = W.fp32_scale(spec.D)

    def step():
        gqa.attn_prefill_paged(q, kc, vc, qo, kvp, idx, inp.max_q_len, kv_last_page_len=last,
                               causal=spec.causal, scale=scale, out=o, lse=lse)

    wall, kern_s, per = time_launches(step, steps, warmup)
    q_lens = (inp.qo_indptr[1:] - inp.qo_indptr[:-1]).tolist()
    n_pages = (inp.kv_indptr[1:] - inp.kv_indptr[:-1]).tolist()
    kv_lens = [0 if n == 0 else (n - 1) * spec.page_size + int(lp)
               for n, lp in zip(n_pages, inp.kv_last_page_len.tolist())]
    flops = 4 * spec.D * spec.Hq * sum(visible_pairs(a, b, spec.causal) for a, b in zip(q_lens, kv_lens))
    return {
        "workload": spec.name, "dtype": spec.dtype, "causal": spec.causal,
        "shape": {"B": spec.B, "Hq": spec.Hq, "Hkv": spec.Hkv, "D": spec.D, "page_size": spec.page_size,
                  "total_q": int(sum(q_lens)), "sum_kv_len": int(sum(kv_lens))},
        "flop_per_launch": flops,
        "ms_per_step": wall / steps * 1e3,
        "kernel_ms_mean": kern_s * 1e3, "call_span_ms_min": float(per.min()) * 1e3,
        "tflops": flops * steps / wall / 1e12,
        "kernel_tflops": flops / kern_s / 1e12,
        "peak_tflops": PEAK_MFMA_16BIT_TFLOPS,
        "frac_of_peak": flops / kern_s / 1e12 / PEAK_MFMA_16BIT_TFLOPS,
    }


def bench_copy(steps, warmup):
    """Calibration for the hardware byte counters: a plain device-to-device copy
    of COPY_BYTES (read COPY_BYTES, write COPY_BYTES) per call."""
    dev = torch.device("cuda:0")
    x = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).uniform_()
    y = torch.empty_like(x)
    wall, kern_s, per = time_launches(lambda: y.copy_(x), steps, warmup)
    return {"workload": "hbm_copy", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
            "kernel_ms_mean": kern_s * 1e3, "gbps": 2 * COPY_BYTES / kern_s / 1e9}


def bench_decode(spec, steps, warmup):
    inp = W.make_decode_spec(spec)
    dev = torch.device("cuda:0")
    q = inp.q.to(dev)
    kc, vc = inp.k_cache.to(dev), inp.v_cache.to(dev)
    sl, bt = inp.seq_lens.to(dev), inp.block_table.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    ws = torch.empty(gqa.decode_workspace_bytes_multi(spec.B, spec.Hq, spec.q_len, spec.D, spec.n_splits),
                     dtype=torch.uint8, device=dev)
    scale = W.fp32_scale(spec.D)
    call = gqa.attn_decode_splitk if spec.q_len == 1 else gqa.attn_decode_splitk_multi

    def step():
        call(q, kc, vc, sl, block_table=bt, n_splits=spec.n_splits, scale=scale,
             max_kv_len=inp.max_kv_len, workspace=ws, out=o, lse=lse)

    wall, kern_s, per = time_launches(step, steps, warmup)
    nbytes = decode_bytes(spec, inp)
    return {
        "workload": spec.name, "dtype": spec.dtype,
        "shape": {"B": spec.B, "Hq": spec.Hq, "Hkv": spec.Hkv, "D": spec.D, "q_len": spec.q_len,
                  "page_size": spec.page_size, "n_splits": spec.n_splits,
                  "sum_kv_len": int(inp.seq_lens.to(torch.int64).sum())},
        "bytes_per_step": nbytes,
        "workspace_bytes_rw": 2 * spec.B * spec.Hq * spec.q_len * spec.n_splits * (spec.D + 1) * 4,
        "ms_per_step": wall / steps * 1e3,
        "kernel_ms_mean": kern_s * 1e3, "call_span_ms_min": float(per.min()) * 1e3,
        "gbps": nbytes * steps / wall / 1e9,
        "kernel_gbps": nbytes / kern_s / 1e9,
        "peak_gbps": PEAK_HBM_GBPS,
        "frac_of_peak": nbytes / kern_s / 1e9 / PEAK_HBM_GBPS,
    }


def _evenly(total: int, n: int) -> np.ndarray:
    return np.unique(np.linspace(0, total - 1, max(1, min(total, n))).astype(np.int64))


def _time_oracle(run_rows, total_rows, row_work, target_s, probe_n=256):
    """Time the oracle on evenly spaced rows: a probe sizes the sample so that
    it takes about target_s seconds.  Returns (work of the sampled rows,
    seconds, rows sampled)."""
    rows = _evenly(total_rows, probe_n)
    t0 = time.perf_counter()
    run_rows(rows)
    dt = time.perf_counter() - t0
    rows = _evenly(total_rows, int(probe_n * target_s / max(dt, 1e-3)))
    t0 = time.perf_counter()
    run_rows(rows)
    dt = time.perf_counter() - t0
    return row_work(rows), dt, len(rows)


def cpu_baseline(spec, target_s=12.0):
    """The oracle, as it stands, timed on the host's cores on a bounded sample
    of the workload's rows (evenly spaced over all of them), its rate in the
    workload's own unit: TFLOP/s on the visible-pair flop count (prefill) or
    GB/s on the step's algorithmic bytes, prorated by the keys each sampled
    row reads (decode)."""
    import oracle
    if isinstance(spec, W.MergeBwdSpec):
        op, lp, d_o, d_lse = (t.numpy() for t in W.make_merge_backward_spec(spec))
        row_bytes = merge_backward_bytes(spec) / spec.rows

        def timed(rows):   # the backward alone; its merged inputs are formed first, untimed
            o_l = oracle.splitk_merge(op[rows], lp[rows])
            t0 = time.perf_counter()
            oracle.splitk_merge_backward(op[rows], lp[rows], o_l[0], o_l[1], d_o[rows], d_lse[rows])
            return time.perf_counter() - t0

        rows = _evenly(spec.rows, 2048)
        dt = timed(rows)
        rows = _evenly(spec.rows, int(2048 * target_s / max(dt, 1e-3)))
        dt = timed(rows)
        n, total = len(rows), spec.rows
        value, unit = row_bytes * n / dt / 1e9, "GB/s"
        return {
            "value": value, "unit": unit, "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{n} of {total} rows of {spec.name} (evenly spaced), fp64, {dt:.1f} s on "
                      f"{oracle.num_threads()} OpenMP threads ({platform.processor() or 'host CPU'})",
        }
    scale = W.fp32_scale(spec.D)
    if spec is W.BIAS_PAGED_DECODE:
        inp, bias = W.make_decode_bias_spec(spec)
        q4 = inp.q.reshape(spec.B, spec.Hq, spec.q_len, spec.D)
        total = spec.B * spec.Hq * spec.q_len
        lens = inp.seq_lens.to(torch.int64).numpy()
        row_len = lens[np.arange(total) // (spec.Hq * spec.q_len)]
        step_bytes = decode_bytes(spec, inp) + decode_bias_bytes(spec, inp)

        def run_rows(rows):
            oracle.attn_decode_bias(q4, inp.k_cache, inp.v_cache, inp.seq_lens, bias, scale,
                                    block_table=inp.block_table, max_kv_len=inp.max_kv_len, rows=rows)

        work, dt, n = _time_oracle(run_rows, total, lambda r: step_bytes * row_len[r].sum() / row_len.sum(),
                                   target_s)
        value, unit = work / dt / 1e9, "GB/s"
    elif spec is W.BIAS_CAUSAL_GQA_PREFILL:
        q, k, v, bias = W.make_prefill_bias_spec(spec)
        total = spec.B * spec.Hq * spec.q_len
        pos = np.arange(total) % spec.q_len
        delta = spec.kv_len - spec.q_len
        vis = np.minimum(spec.kv_len, np.maximum(0, pos + 1 + delta)) if spec.causal else \
            np.full_like(pos, spec.kv_len)
        row_flops = 4 * spec.D * vis
        work, dt, n = _time_oracle(lambda r: oracle.attn_fwd_bias(q, k, v, bias, scale, spec.causal, rows=r),
                                   total, lambda r: row_flops[r].sum(), target_s)
        value, unit = work / dt / 1e12, "TFLOP/s"
    elif isinstance(spec, W.DecodeSpec) or spec is W.FP8_PAGED_DECODE:
        fp8 = spec is W.FP8_PAGED_DECODE
        inp = W.make_decode_fp8_spec(spec) if fp8 else W.make_decode_spec(spec)
        q_len = 1 if fp8 else spec.q_len
        total = spec.B * spec.Hq * q_len
        lens = inp.seq_lens.to(torch.int64).numpy()
        row_len = lens[np.arange(total) // (spec.Hq * q_len)]
        step_bytes = decode_bytes(spec, inp, fp8=fp8)

        def run_rows(rows):
            if fp8:
                oracle.attn_decode_fp8(inp.q, inp.k8, inp.v8, inp.k_ss, inp.v_ss, inp.seq_lens, scale,
                                       block_table=inp.block_table, max_kv_len=inp.max_kv_len, rows=rows)
            elif q_len == 1:
                oracle.attn_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, scale,
                                   block_table=inp.block_table, max_kv_len=inp.max_kv_len, rows=rows)
            else:
                oracle.attn_decode_multi(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, scale,
                                         block_table=inp.block_table, max_kv_len=inp.max_kv_len, rows=rows)

        work, dt, n = _time_oracle(run_rows, total, lambda r: step_bytes * row_len[r].sum() / row_len.sum(),
                                   target_s)
        value, unit = work / dt / 1e9, "GB/s"
    elif isinstance(spec, W.PagedPrefillSpec):
        inp = W.make_paged_prefill_spec(spec)
        qo = inp.qo_indptr.to(torch.int64).numpy()
        n_pages = (inp.kv_indptr[1:] - inp.kv_indptr[:-1]).to(torch.int64).numpy()
        last = inp.kv_last_page_len.to(torch.int64).numpy()
        kv = np.where(n_pages > 0, (n_pages - 1) * spec.page_size + last, 0)
        tok = np.arange(qo[-1])
        req = np.searchsorted(qo, tok, side="right") - 1
        i = tok - qo[req]
        qn = qo[req + 1] - qo[req]
        vis = np.minimum(kv[req], np.maximum(0, i + 1 + kv[req] - qn)) if spec.causal else kv[req]
        row_flops = np.repeat(4 * spec.D * vis, spec.Hq)   # flat row = token * Hq + head

        def run_rows(rows):
            oracle.attn_prefill_paged(inp.q, inp.k_cache, inp.v_cache, inp.qo_indptr, inp.kv_indptr,
                                      inp.kv_indices, scale, spec.causal, inp.kv_last_page_len, rows=rows)

        work, dt, n = _time_oracle(run_rows, len(row_flops), lambda r: row_flops[r].sum(), target_s)
        total = len(row_flops)
        value, unit = work / dt / 1e12, "TFLOP/s"
    else:
        q, k, v = W.make_prefill_spec(spec)
        total = spec.B * spec.Hq * spec.q_len
        pos = np.arange(total) % spec.q_len
        delta = spec.kv_len - spec.q_len
        vis = np.minimum(spec.kv_len, np.maximum(0, pos + 1 + delta)) if spec.causal else \
            np.full_like(pos, spec.kv_len)
        row_flops = 4 * spec.D * vis
        work, dt, n = _time_oracle(lambda r: oracle.attn_fwd(q, k, v, scale, spec.causal, rows=r), total,
                                   lambda r: row_flops[r].sum(), target_s)
        value, unit = work / dt / 1e12, "TFLOP/s"
    return {
        "value": value, "unit": unit, "cores": oracle.num_threads(), "kind": "oracle",
        "sample": f"{n} of {total} rows of {spec.name} (evenly spaced), fp64, {dt:.1f} s on "
                  f"{oracle.num_threads()} OpenMP threads ({platform.processor() or 'host CPU'})",
    }


def _n_cu() -> int:
    return torch.cuda.get_device_properties(0).multi_processor_count


def bench_mfma_ceiling(steps, warmup):
    """The MFMA-only loop (include/gqa_ceilings.h) at the prefill kernel's
    occupancy: the matrix-core rate the chip sustains under a full load."""
    n_wg, iters = 4 * _n_cu(), 1000
    out = torch.empty(n_wg * 512, dtype=torch.float32, device="cuda:0")
    flops = gqa.ceiling_mfma(n_wg, iters, out)[0]
    wall, kern_s, per = time_launches(lambda: gqa.ceiling_mfma(n_wg, iters, out), steps, warmup)
    return {"workload": "mfma_ceiling", "what": "v_mfma_f32_32x32x16_bf16 back to back, 8 waves per CU, "
            "no memory traffic", "flop_per_launch": flops, "kernel_ms_mean": kern_s * 1e3,
            "tflops": flops / kern_s / 1e12, "peak_tflops": PEAK_MFMA_16BIT_TFLOPS,
            "frac_of_peak": flops / kern_s / 1e12 / PEAK_MFMA_16BIT_TFLOPS}


READ_CEILING_BYTES = 1 << 30


def bench_read_ceiling(steps, warmup):
    """The streaming read (include/gqa_ceilings.h) over 1 GiB, four times the
    last-level cache: the rate HBM gives a pure read stream."""
    src = torch.empty(READ_CEILING_BYTES // 4, dtype=torch.int32, device="cuda:0").random_()
    n_wg = 32 * _n_cu()
    out = torch.empty(n_wg, dtype=torch.int32, device="cuda:0")
    wall, kern_s, per = time_launches(lambda: gqa.ceiling_stream_read(src, n_wg, out), steps, warmup)
    return {"workload": "hbm_read_ceiling", "what": "16-byte non-temporal loads, every byte of 1 GiB once",
            "bytes_per_launch": READ_CEILING_BYTES, "kernel_ms_mean": kern_s * 1e3,
            "gbps": READ_CEILING_BYTES / kern_s / 1e9, "peak_gbps": PEAK_HBM_GBPS,
            "frac_of_peak": READ_CEILING_BYTES / kern_s / 1e9 / PEAK_HBM_GBPS}


def run_one(spec, steps, warmup):
    if spec is W.BIAS_CAUSAL_GQA_PREFILL:
        return bench_prefill_bias(spec, steps, warmup)
    if spec is W.BIAS_PAGED_DECODE:
        return bench_decode_bias(spec, steps, warmup)
    if isinstance(spec, W.MergeBwdSpec):
        return bench_merge_backward(spec, steps, warmup)
    if spec is W.FP8_PAGED_DECODE:
        return bench_decode_fp8(spec, steps, warmup)
    if isinstance(spec, W.DecodeSpec):
        return bench_decode(spec, steps, warmup)
    if isinstance(spec, W.PagedPrefillSpec):
        return bench_paged_prefill(spec, steps, warmup)
    return bench_prefill(spec, steps, warmup)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="time only this workload (profiling runs); 'hbm_copy' times a plain copy "
                         "used to calibrate the HBM byte counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "one GPU only: run with --gpus 1 (several GPUs would each run the "
                                   "same kernels on their share; that sharding is not implemented)"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)

    all_specs = [W.CAUSAL_GQA_FP32, W.CAUSAL_GQA_PREFILL, W.CAUSAL_GQA_OFFSET,
                 W.MHA_NONCAUSAL_FP16, W.PAGED_DECODE, W.FP8_PAGED_DECODE, W.MULTI_QUERY_DECODE,
                 W.RAGGED_PAGED_PREFILL, W.BIAS_CAUSAL_GQA_PREFILL, W.BIAS_PAGED_DECODE,
                 W.SPLITK_MERGE_BACKWARD]
    ceilings = {"mfma_ceiling": bench_mfma_ceiling, "hbm_read_ceiling": bench_read_ceiling}
    if args.only == "hbm_copy":
        print(json.dumps(bench_copy(args.steps, args.warmup)), flush=True)
        return
    if args.only in ceilings:
        print(json.dumps(ceilings[args.only](args.steps, args.warmup)), flush=True)
        return
    if args.only:
        specs = [s for s in all_specs if s.name == args.only]
        if not specs:
            sys.exit(f"unknown workload {args.only}")
        for s in specs:
            print(json.dumps(run_one(s, args.steps, args.warmup)), flush=True)
        return

    results = {}
    for s in all_specs:
        if s is PRIMARY:
            continue
        r = run_one(s, max(20, args.steps // 2), args.warmup)
        results[s.name] = r
        print(f"# {s.name}: {json.dumps(r)}", file=sys.stderr, flush=True)
    ceil = {name: fn(20, 3) for name, fn in ceilings.items()}
    print(f"# ceilings: {json.dumps(ceil)}", file=sys.stderr, flush=True)
    mfma_ceil, read_ceil = ceil["mfma_ceiling"]["tflops"], ceil["hbm_read_ceiling"]["gbps"]
    for r in results.values():
        if "kernel_tflops" in r and r.get("dtype") != "f32":
            r["frac_of_measured_mfma_ceiling"] = r["kernel_tflops"] / mfma_ceil
        if "kernel_gbps" in r:
            r["frac_of_measured_read_ceiling"] = r["kernel_gbps"] / read_ceil

    torch.cuda.synchronize()
    p = bench_prefill(PRIMARY, args.steps, args.warmup)
    results[PRIMARY.name] = p
    line = {
        "metric": METRIC,
        "value": round(p["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(p["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": PRIMARY.name, "B": PRIMARY.B, "Hq": PRIMARY.Hq, "Hkv": PRIMARY.Hkv,
                   "seq_len": PRIMARY.q_len, "D": PRIMARY.D, "causal": True,
                   "global_batch": PRIMARY.B, "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(p["kernel_tflops"], 3),
            "peak": PEAK_MFMA_16BIT_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(p["frac_of_peak"], 4),
            "traffic": measured_traffic(),
            "kernel": "prefill_fwd_pp<bf16, D=128, causal, 4 heads/workgroup>",
            "kernel_ms_mean": round(p["kernel_ms_mean"], 5),
            "measured_ceiling": {"value": round(mfma_ceil, 3), "unit": "TFLOP/s",
                                 "what": ceil["mfma_ceiling"]["what"],
                                 "frac": round(p["kernel_tflops"] / mfma_ceil, 4)},
        },
        "ceilings": ceil,
        "workloads": results,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(PRIMARY)
        for s in all_specs:
            if s is not PRIMARY:
                results[s.name]["cpu_baseline"] = cpu_baseline(s, target_s=3.0)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
