"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out: it holds none of the
attention arithmetic, and it imports neither the HIP binding nor the oracle.
Every tensor is drawn on the CPU from ``torch.Generator().manual_seed(seed)``,
in fp32 from N(0, 1), optionally multiplied by an exact power of two, and then
rounded (round-to-nearest-even) to the storage dtype.  The rounded host copy
is what both the GPU and the oracle consume.

Workloads (shapes of the attention problems the pages state):
  causal_gqa_fp32       B=1 Hq=4 Hkv=2 S=128 D=64, fp32, causal
  causal_gqa_prefill    B=2 Hq=32 Hkv=8 S=2048 D=128, bf16, causal
  causal_gqa_offset     B=1 Hq=32 Hkv=4 q_len=1024 kv_len=4096 D=128, bf16,
                        causal with the bottom-right offset (delta = 3072)
  mha_noncausal_fp16    B=4 H=16 S=4096 D=64, fp16, inputs x0.5, non-causal
  paged_decode          B=16 Hq=32 Hkv=8 D=128, bf16, kv_len ~ U[1024, 32768],
                        256-token pages placed by a seeded permutation, 16 splits
  multi_query_decode    the same with 4 queries per sequence at its last positions
  fp8_paged_decode      paged_decode over an 8-bit E4M3 K/V cache with a binary16
                        (scale, shift) pair per token row and K/V head
  ragged_paged_prefill  8 requests, Hq=32 Hkv=4 D=128, bf16, causal; request b has
                        q_len ~ U[256, 2048] new tokens after a cached prefix of
                        U[0, 2048] tokens; one token per page, pages placed by a
                        seeded permutation; q token-major [total_q, Hq, D]
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def fp32_scale(D: int) -> float:
    """1/sqrt(D) rounded to fp32: the exact scale value both sides receive."""
    return float(np.float32(1.0 / math.sqrt(D)))


@dataclass(frozen=True)
class PrefillSpec:
    name: str
    B: int
    Hq: int
    Hkv: int
    q_len: int
    kv_len: int
    D: int
    dtype: str
    causal: bool
    seed: int
    mult: float = 1.0


@dataclass(frozen=True)
class DecodeSpec:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    len_lo: int
    len_hi: int          # inclusive
    page_size: int
    max_pages: int
    n_splits: int
    seed: int
    q_len: int = 1       # queries per sequence (its last positions); 1 is plain decode


CAUSAL_GQA_FP32 = PrefillSpec("causal_gqa_fp32", 1, 4, 2, 128, 128, 64, "f32", True, 20261)
CAUSAL_GQA_PREFILL = PrefillSpec("causal_gqa_prefill", 2, 32, 8, 2048, 2048, 128, "bf16", True, 20262)
CAUSAL_GQA_OFFSET = PrefillSpec("causal_gqa_offset", 1, 32, 4, 1024, 4096, 128, "bf16", True, 20263)
MHA_NONCAUSAL_FP16 = PrefillSpec("mha_noncausal_fp16", 4, 16, 16, 4096, 4096, 64, "f16", False, 20264, 0.5)
PAGED_DECODE = DecodeSpec("paged_decode", 16, 32, 8, 128, "bf16", 1024, 32768, 256, 128, 16, 20265)
FP8_PAGED_DECODE = DecodeSpec("fp8_paged_decode", 16, 32, 8, 128, "bf16", 1024, 32768, 256, 128, 16, 20268)
MULTI_QUERY_DECODE = DecodeSpec("multi_query_decode", 16, 32, 8, 128, "bf16", 1024, 32768, 256, 128, 16,
                                20266, q_len=4)

PREFILL_WORKLOADS = [CAUSAL_GQA_FP32, CAUSAL_GQA_PREFILL, CAUSAL_GQA_OFFSET, MHA_NONCAUSAL_FP16]


@dataclass(frozen=True)
class PagedPrefillSpec:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    q_lo: int            # new query tokens per request ~ U[q_lo, q_hi]
    q_hi: int
    prefix_lo: int       # cached tokens before them ~ U[prefix_lo, prefix_hi]
    prefix_hi: int
    page_size: int
    causal: bool
    seed: int


# Batched prefill over a paged cache with the head geometry of the FlashInfer-style
# prefill page (32 query heads, 4 K/V heads, D = 128, one token per page).
RAGGED_PAGED_PREFILL = PagedPrefillSpec("ragged_paged_prefill", 8, 32, 4, 128, "bf16", 256, 2048, 0, 2048,
                                        1, True, 20267)


def _randn(shape, g, dtype, mult=1.0):
    x = torch.randn(shape, dtype=torch.float32, generator=g)
    if mult != 1.0:
        x.mul_(mult)  # the multipliers used are powers of two: exact in fp32
    return x.to(dtype)


def make_prefill(B, Hq, Hkv, q_len, kv_len, D, dtype="bf16", seed=0, mult=1.0):
    """Q [B,Hq,q_len,D], K/V [B,Hkv,kv_len,D] on the CPU, drawn in the order Q, K, V."""
    g = torch.Generator().manual_seed(seed)
    dt = _DTYPES[dtype]
    q = _randn((B, Hq, q_len, D), g, dt, mult)
    k = _randn((B, Hkv, kv_len, D), g, dt, mult)
    v = _randn((B, Hkv, kv_len, D), g, dt, mult)
    return q, k, v


def make_prefill_spec(spec: PrefillSpec):
    return make_prefill(spec.B, spec.Hq, spec.Hkv, spec.q_len, spec.kv_len, spec.D,
                        spec.dtype, spec.seed, spec.mult)


@dataclass
class DecodeInputs:
    q: torch.Tensor            # [B, Hq, D], or [B, Hq, q_len, D] when q_len is given
    k_cache: torch.Tensor      # [num_pages, page_size, Hkv, D]
    v_cache: torch.Tensor
    seq_lens: torch.Tensor     # [B] int32
    block_table: torch.Tensor  # [B, max_pages] int32, -1 padding
    page_size: int
    max_kv_len: int


def make_decode(B, Hq, Hkv, D, dtype="bf16", seed=0, len_lo=1, len_hi=64, page_size=256,
                max_pages: Optional[int] = None, seq_lens=None, permute=True, q_len: Optional[int] = None):
    """Paged decode inputs, drawn in the order q, seq_lens, page permutation, K, V.

    Sequence b uses n_b = ceil(len_b / page_size) pages; pages are handed out
    from a seeded permutation of all pages (identity when permute=False) in
    sequence order; unused block-table slots hold -1.
    """
    g = torch.Generator().manual_seed(seed)
    dt = _DTYPES[dtype]
    q = _randn((B, Hq, D) if q_len is None else (B, Hq, q_len, D), g, dt)
    if seq_lens is None:
        seq_lens = torch.randint(len_lo, len_hi + 1, (B,), generator=g, dtype=torch.int64)
    seq_lens = torch.as_tensor(seq_lens, dtype=torch.int64)
    n_pages = [(int(s) + page_size - 1) // page_size for s in seq_lens]
    total_pages = max(1, sum(n_pages))
    perm = torch.randperm(total_pages, generator=g) if permute else torch.arange(total_pages)
    if max_pages is None:
        max_pages = max(1, max(n_pages) if n_pages else 1)
    bt = torch.full((B, max_pages), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(n_pages):
        if n > max_pages:
            raise ValueError("sequence needs more pages than max_pages")
        bt[b, :n] = perm[off:off + n].to(torch.int32)
        off += n
    k = _randn((total_pages, page_size, Hkv, D), g, dt)
    v = _randn((total_pages, page_size, Hkv, D), g, dt)
    return DecodeInputs(q, k, v, seq_lens.to(torch.int32), bt, page_size, max_pages * page_size)


def make_decode_spec(spec: DecodeSpec):
    return make_decode(spec.B, spec.Hq, spec.Hkv, spec.D, spec.dtype, spec.seed,
                       spec.len_lo, spec.len_hi, spec.page_size, spec.max_pages,
                       q_len=None if spec.q_len == 1 else spec.q_len)



@dataclass
class PagedPrefillInputs:
    q: torch.Tensor                  # [total_q, Hq, D]
    k_cache: torch.Tensor            # [num_pages, page_size, Hkv, D]
    v_cache: torch.Tensor
    qo_indptr: torch.Tensor          # [B + 1] int32
    kv_indptr: torch.Tensor          # [B + 1] int32 (page offsets into kv_indices)
    kv_indices: torch.Tensor         # [nnz_pages] int32
    kv_last_page_len: torch.Tensor   # [B] int32 (tokens in each request's last page)
    page_size: int
    max_q_len: int


def make_paged_prefill(B, Hq, Hkv, D, dtype="bf16", seed=0, q_lo=1, q_hi=64, prefix_lo=0, prefix_hi=64,
                       page_size=16, q_lens=None, kv_lens=None, permute=True):
    """Ragged prefill inputs over a paged pool, drawn in the order q_lens,
    prefix lengths, q, page permutation, K, V (q_lens / kv_lens may be given).

    Request b has q_lens[b] new tokens and kv_lens[b] keys (its cached prefix
    and its own tokens, kv_len = prefix + q_len by default); its
    ceil(kv_len / page_size) pages are handed out from a seeded permutation of
    all pages in request order.
    """
    g = torch.Generator().manual_seed(seed)
    dt = _DTYPES[dtype]
    if q_lens is None:
        q_lens = torch.randint(q_lo, q_hi + 1, (B,), generator=g, dtype=torch.int64)
    q_lens = torch.as_tensor(q_lens, dtype=torch.int64)
    if kv_lens is None:
        prefix = torch.randint(prefix_lo, prefix_hi + 1, (B,), generator=g, dtype=torch.int64)
        kv_lens = q_lens + prefix
    kv_lens = torch.as_tensor(kv_lens, dtype=torch.int64)
    total_q = int(q_lens.sum())
    q = _randn((total_q, Hq, D), g, dt)
    n_pages = [(int(n) + page_size - 1) // page_size for n in kv_lens]
    total_pages = max(1, sum(n_pages))
    perm = torch.randperm(total_pages, generator=g) if permute else torch.arange(total_pages)
    k = _randn((total_pages, page_size, Hkv, D), g, dt)
    v = _randn((total_pages, page_size, Hkv, D), g, dt)
    qo = torch.zeros(B + 1, dtype=torch.int32)
    qo[1:] = torch.cumsum(q_lens, 0).to(torch.int32)
    kvp = torch.zeros(B + 1, dtype=torch.int32)
    kvp[1:] = torch.cumsum(torch.as_tensor(n_pages, dtype=torch.int64), 0).to(torch.int32)
    idx = perm[:sum(n_pages)].to(torch.int32)
    last = torch.tensor([int(n) - (p - 1) * page_size if p > 0 else 0 for n, p in zip(kv_lens, n_pages)],
                        dtype=torch.int32)
    return PagedPrefillInputs(q, k, v, qo, kvp, idx, last, page_size, max(1, int(q_lens.max()) if B else 1))


def make_paged_prefill_spec(spec: PagedPrefillSpec):
    return make_paged_prefill(spec.B, spec.Hq, spec.Hkv, spec.D, spec.dtype, spec.seed, spec.q_lo, spec.q_hi,
                              spec.prefix_lo, spec.prefix_hi, spec.page_size)


@dataclass
class DecodeFp8Inputs:
    q: torch.Tensor            # [B, Hq, D] (bf16 / fp16)
    k8: torch.Tensor           # [num_pages, page_size, Hkv, D] uint8 (E4M3 bytes)
    v8: torch.Tensor
    k_ss: torch.Tensor         # [num_pages, page_size, Hkv] int32: fp16 scale bits 0-15, shift bits 16-31
    v_ss: torch.Tensor
    seq_lens: torch.Tensor     # [B] int32
    block_table: torch.Tensor  # [B, max_pages] int32, -1 padding
    page_size: int
    max_kv_len: int


def quantize_e4m3_rows(x: torch.Tensor):
    """Per row (last dimension): shift = row mean and scale = max |x - shift| / 448,
    both rounded to fp16; bytes = E4M3(x - shift) / scale), rounded by torch's
    cast.  Returns (uint8 bytes, int32 words with the scale in bits 0-15 and the
    shift in bits 16-31)."""
    shift = x.mean(dim=-1, keepdim=True).to(torch.float16)
    dev = (x - shift.float()).abs().amax(dim=-1, keepdim=True)
    scale = torch.where(dev > 0, dev / 448.0, torch.ones_like(dev)).to(torch.float16)
    q8 = ((x - shift.float()) / scale.float()).to(torch.float8_e4m3fn).view(torch.uint8)
    sb = scale.view(torch.int16).to(torch.int32) & 0xFFFF
    hb = shift.view(torch.int16).to(torch.int32) & 0xFFFF
    return q8, (sb | (hb << 16)).squeeze(-1)


def make_decode_fp8(B, Hq, Hkv, D, dtype="bf16", seed=0, len_lo=1, len_hi=64, page_size=256,
                    max_pages: Optional[int] = None, seq_lens=None, permute=True):
    """Paged decode inputs with an E4M3 K/V cache: drawn like make_decode (q,
    seq_lens, page permutation, K, V in fp32 N(0, 1)), then every (token, head)
    row of K and V quantized by quantize_e4m3_rows."""
    base = make_decode(B, Hq, Hkv, D, "f32", seed, len_lo, len_hi, page_size, max_pages, seq_lens, permute)
    k8, kss = quantize_e4m3_rows(base.k_cache)
    v8, vss = quantize_e4m3_rows(base.v_cache)
    return DecodeFp8Inputs(base.q.to(_DTYPES[dtype]), k8, v8, kss, vss, base.seq_lens, base.block_table,
                           page_size, base.max_kv_len)


def make_decode_fp8_spec(spec: DecodeSpec):
    return make_decode_fp8(spec.B, spec.Hq, spec.Hkv, spec.D, spec.dtype, spec.seed, spec.len_lo, spec.len_hi,
                           spec.page_size, spec.max_pages)


# ---- additive bias and split-K merge backward ------------------------------------

# The headline prefill shape with a per-head additive bias [1, Hq, q_len, kv_len]
# (shared by the batch, like a relative-position bias), and the paged decode
# shape with a bias per (sequence, head) over its keys [B, Hq, 1, max_kv_len]
# (the HAS_ADDITIVE_BIAS operand of the split-K decode page).
BIAS_CAUSAL_GQA_PREFILL = PrefillSpec("bias_causal_gqa_prefill", 2, 32, 8, 2048, 2048, 128, "bf16", True, 20270)
BIAS_PAGED_DECODE = DecodeSpec("bias_paged_decode", 16, 32, 8, 128, "bf16", 1024, 32768, 256, 128, 16, 20271)


@dataclass(frozen=True)
class MergeBwdSpec:
    name: str
    rows: int            # merged rows (query, head)
    n_splits: int
    D: int
    empty: int           # partials with no visible key (LSE -inf), placed at random
    seed: int


# Backward of the merge of the split-KV prefill's partials at the bottom-right
# offset shape (B=1, Hq=32, q_len=1024: 32768 rows, 4 key ranges, D=128).
SPLITK_MERGE_BACKWARD = MergeBwdSpec("splitk_merge_backward", 32768, 4, 128, 256, 20272)


def make_bias(shape, dtype="bf16", seed=0, mult=2.0):
    """An additive bias of `shape`, N(0, 1) * mult rounded to dtype."""
    g = torch.Generator().manual_seed(seed)
    return _randn(shape, g, _DTYPES[dtype], mult)


def make_prefill_bias_spec(spec: PrefillSpec):
    """q, k, v of the prefill shape and a per-head bias [1, Hq, q_len, kv_len]."""
    q, k, v = make_prefill_spec(spec)
    return q, k, v, make_bias((1, spec.Hq, spec.q_len, spec.kv_len), spec.dtype, spec.seed + 1)


def make_decode_bias_spec(spec: DecodeSpec):
    """Paged decode inputs (make_decode_spec) and a bias [B, Hq, q_len, max_kv_len]."""
    inp = make_decode_spec(spec)
    return inp, make_bias((spec.B, spec.Hq, spec.q_len, inp.max_kv_len), spec.dtype, spec.seed + 1)


def make_merge_backward_spec(spec: MergeBwdSpec):
    """Partials of a split-K merge and the gradients of a scalar with respect to
    its outputs, fp32: o_parts [rows, S, D] ~ N(0, 1), lse_parts [rows, S] ~
    3 N(0, 1) with `empty` partials set to (0, -inf) and row 0 empty in every
    range, d_o [rows, D] and d_lse [rows] ~ N(0, 1).  The merged (o, lse) the
    backward also takes are the merge of these partials."""
    g = torch.Generator().manual_seed(spec.seed)
    op = torch.randn((spec.rows, spec.n_splits, spec.D), generator=g)
    lp = 3.0 * torch.randn((spec.rows, spec.n_splits), generator=g)
    r = torch.randint(0, spec.rows, (spec.empty,), generator=g)
    s = torch.randint(0, spec.n_splits, (spec.empty,), generator=g)
    op[r, s] = 0.0
    lp[r, s] = float("-inf")
    op[0] = 0.0
    lp[0] = float("-inf")
    d_o = torch.randn((spec.rows, spec.D), generator=g)
    d_lse = torch.randn((spec.rows,), generator=g)
    return op, lp, d_o, d_lse
