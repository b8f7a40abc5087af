"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances (max abs error over the compared elements):
  fp32 inputs         O and LSE within 1e-5
  bf16 / fp16 inputs  O within 2e-2, LSE within 1e-3
A -inf LSE must be -inf on both sides and no NaN may appear anywhere.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import gqa_attention_forward_attn_amd as gqa
import workloads as W

pytestmark = pytest.mark.gpu

# every block table and CSR pointer set a test passes is also checked on the
# host before the launch (the kernels themselves trust them)
gqa.set_check_tables(True)

TOL = {"f32": (1e-5, 1e-5), "bf16": (2e-2, 1e-3), "f16": (2e-2, 1e-3)}
DTNAME = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtname, what=""):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    tol_o, tol_l = TOL[dtname]
    assert not np.isnan(o_gpu).any(), f"{what}: NaN in O"
    assert not np.isnan(lse_gpu).any(), f"{what}: NaN in LSE"
    err_o = np.abs(o_gpu - o_ref).max() if o_ref.size else 0.0
    assert err_o <= tol_o, f"{what}: max |O - oracle| = {err_o:.3e} > {tol_o}"
    ninf_ref = np.isneginf(lse_ref)
    assert np.array_equal(ninf_ref, np.isneginf(lse_gpu)), f"{what}: -inf LSE pattern differs"
    fin = ~ninf_ref
    err_l = np.abs(lse_gpu[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    assert err_l <= tol_l, f"{what}: max |LSE - oracle| = {err_l:.3e} > {tol_l}"
    return err_o, err_l


def gpu_fwd(q, k, v, causal, scale, canary=True, kv_splits=1, kernel=None):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.full_like(qd, float("nan")) if canary else None
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda") if canary else None
    o, l = gqa.attn_fwd(qd, kd, vd, causal=causal, scale=scale, out=out, lse=lse, kv_splits=kv_splits,
                        kernel=kernel)
    torch.cuda.synchronize()
    return o, l


# ---- prefill: every element, several tiles and ragged tails ----------------

SMALL = [
    # B, Hq, Hkv, q_len, kv_len, D, dtype, causal
    (1, 4, 2, 128, 128, 64, "f32", True),
    (2, 4, 2, 200, 200, 64, "f32", False),
    (1, 2, 1, 70, 300, 128, "f32", True),
    (2, 8, 2, 200, 200, 128, "bf16", True),
    (1, 8, 8, 130, 333, 64, "f16", False),
    (1, 8, 1, 77, 300, 128, "bf16", True),     # bottom-right offset, G = 8
    (2, 4, 2, 300, 100, 64, "bf16", True),     # q_len > kv_len: leading rows empty
    (1, 2, 2, 1, 517, 128, "bf16", True),      # single query row
    (1, 6, 3, 257, 257, 128, "f16", True),     # G = 2
    (3, 4, 4, 65, 1, 64, "bf16", False),       # one key
    (1, 32, 4, 96, 416, 128, "bf16", True),    # G = 8 with offset
    (1, 12, 4, 64, 64, 64, "f16", True),       # G = 3
]


# bf16 / fp16 prefill has two kernels (chosen by shape); every shape runs on both
PREFILL_KERNELS = ["pingpong", "fourwave"]
SMALL_CASES = [(s, kern) for s in SMALL for kern in (PREFILL_KERNELS if s[6] != "f32" else ["auto"])]


@pytest.mark.parametrize("shape,kernel", SMALL_CASES, ids=lambda c: "-".join(map(str, c)) if isinstance(c, tuple) else c)
def test_prefill_all_elements(shape, kernel):
    B, Hq, Hkv, Lq, Lk, D, dt, causal = shape
    print(f"prefill case {shape} kernel {kernel}", flush=True)
    q, k, v = W.make_prefill(B, Hq, Hkv, Lq, Lk, D, dt, seed=sum(shape[:6]))
    scale = W.fp32_scale(D)
    o, l = gpu_fwd(q, k, v, causal, scale, kernel=kernel)
    o_ref, l_ref = oracle.attn_fwd(q, k, v, scale, causal)
    check(o.double().cpu().numpy(), l.double().cpu().numpy(), o_ref, l_ref, dt, str(shape))


# ---- split-KV prefill: key ranges in parallel, merged by LSE ----------------

SPLIT = [
    # B, Hq, Hkv, q_len, kv_len, D, dtype, causal, kv_splits
    (1, 8, 2, 200, 700, 128, "bf16", True, 2),
    (1, 8, 2, 200, 700, 128, "bf16", True, 3),
    (2, 4, 4, 130, 333, 64, "f16", False, 2),
    (2, 4, 4, 130, 333, 64, "f16", False, 5),
    (1, 32, 4, 96, 2100, 128, "bf16", True, 4),     # bottom-right offset, G = 8
    (2, 4, 2, 300, 100, 64, "bf16", True, 3),       # q_len > kv_len: leading rows see no key
    (1, 6, 3, 257, 257, 128, "f16", True, 8),       # more ranges than some row blocks have tiles
    (1, 12, 4, 64, 64, 64, "bf16", True, 2),        # G = 3, a single key tile
    (1, 8, 2, 200, 1500, 128, "bf16", True, 13),    # more than 8 ranges: the merge takes them in groups
    (1, 4, 4, 64, 2048, 64, "f16", False, 20),      # 16 non-empty ranges, then 4 empty ones
]


@pytest.mark.parametrize("case", SPLIT, ids=lambda c: "-".join(map(str, c)))
def test_prefill_split_all_elements(case):
    B, Hq, Hkv, Lq, Lk, D, dt, causal, S = case
    print(f"split prefill case {case}", flush=True)
    q, k, v = W.make_prefill(B, Hq, Hkv, Lq, Lk, D, dt, seed=sum(case[:6]) + S)
    scale = W.fp32_scale(D)
    o, l = gpu_fwd(q, k, v, causal, scale, kv_splits=S)
    o_ref, l_ref = oracle.attn_fwd(q, k, v, scale, causal)
    check(o.double().cpu().numpy(), l.double().cpu().numpy(), o_ref, l_ref, dt, str(case))
    # the merge of the ranges equals the single pass of the same kernel up to
    # rounding: the tiles and their rounded weights are the same, only the
    # order of the fp32 sums and the final rounding differ
    o1, l1 = gpu_fwd(q, k, v, causal, scale, kv_splits=1, kernel="pingpong")
    lf, l1f = l.cpu(), l1.cpu()
    assert torch.equal(torch.isneginf(lf), torch.isneginf(l1f))
    fin = torch.isfinite(l1f)
    assert float((lf[fin] - l1f[fin]).abs().max()) <= 1e-5
    assert float((o.float() - o1.float()).abs().max()) <= 1.6e-2



# small grids at full length: the library's own range count (2 x the CUs /
# blocks for causal shapes whose offset is below q_len, ranges of >= 8 tiles)
RECOMMENDED_SPLIT = [
    # B, Hq, Hkv, q_len, kv_len
    (2, 4, 1, 2048, 2048),     # one GPU's share of the 2 x 32-head workload over 8 GPUs
    (1, 8, 2, 3072, 3072),     # causal without offset: the doubled count
    (1, 32, 4, 512, 4096),     # offset 3584 >= q_len: not doubled
]


@pytest.mark.parametrize("shape", RECOMMENDED_SPLIT, ids=lambda c: "-".join(map(str, c)))
def test_prefill_recommended_split_small_grid(shape):
    B, Hq, Hkv, Lq, Lk = shape
    S = gqa.lib().attn_fwd_kv_splits(B, Hq, Hkv, Lq, Lk, 128, 1, gqa._TORCH_DT[torch.bfloat16])
    print(f"recommended split {shape}: {S} ranges", flush=True)
    assert S >= 2
    q, k, v = W.make_prefill(B, Hq, Hkv, Lq, Lk, 128, "bf16", seed=Lq + Lk + Hq)
    scale = W.fp32_scale(128)
    o, l = gpu_fwd(q, k, v, True, scale, kv_splits=None)
    o_ref, l_ref = oracle.attn_fwd(q, k, v, scale, True)
    check(o.double().cpu().numpy(), l.double().cpu().numpy(), o_ref, l_ref, "bf16", str(shape))
    o1, l1 = gpu_fwd(q, k, v, True, scale, kv_splits=1, kernel="pingpong")
    assert float((l.cpu() - l1.cpu()).abs().max()) <= 1e-5
    assert float((o.float() - o1.float()).abs().max()) <= 1.6e-2

def test_prefill_kv_len_zero():
    q = torch.randn(1, 4, 16, 64).to(torch.bfloat16)
    k = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16)
    o, l = gpu_fwd(q, k, k.clone(), False, 0.125)
    assert torch.all(o.float() == 0) and torch.all(torch.isneginf(l))


# ---- prefill at the workload sizes: every element ----------------------------
# The oracle runs once per workload (cached for the module) and every kernel
# variant is compared with it on all rows of O and LSE.

_WORKLOAD_ORACLE = {}


def workload_oracle(spec):
    if spec.name not in _WORKLOAD_ORACLE:
        q, k, v = W.make_prefill_spec(spec)
        scale = W.fp32_scale(spec.D)
        _WORKLOAD_ORACLE[spec.name] = (q, k, v, scale, oracle.attn_fwd(q, k, v, scale, spec.causal))
    return _WORKLOAD_ORACLE[spec.name]


WORKLOAD_CASES = [(s, kern) for s in W.PREFILL_WORKLOADS
                  for kern in (PREFILL_KERNELS + ["split"] if s.dtype != "f32" else ["auto"])]


@pytest.mark.parametrize("spec,kernel", WORKLOAD_CASES,
                         ids=lambda c: c.name if hasattr(c, "name") else c)
def test_prefill_workload_all_elements(spec, kernel):
    # "split": key ranges merged by LSE, with the library's range count for the
    # shape (at least 2, so that every workload also runs the split path)
    splits = 1
    if kernel == "split":
        splits = max(2, gqa.lib().attn_fwd_kv_splits(spec.B, spec.Hq, spec.Hkv, spec.q_len, spec.kv_len,
                                                     spec.D, int(spec.causal), gqa._TORCH_DT[W._DTYPES[spec.dtype]]))
    print(f"workload {spec.name} kernel {kernel} kv_splits {splits}", flush=True)
    q, k, v, scale, (o_ref, l_ref) = workload_oracle(spec)
    o, l = gpu_fwd(q, k, v, spec.causal, scale, kv_splits=splits,
                   kernel=kernel if kernel in PREFILL_KERNELS else None)
    e_o, e_l = check(o.double().cpu().numpy(), l.double().cpu().numpy(), o_ref, l_ref, spec.dtype, spec.name)
    print(f"{spec.name} ({kernel}): all {l_ref.size} rows, max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}")


def test_causal_row_zero_exact():
    # delta = 0: row 0 sees key 0 only, so P = 1 and O[0] = V[0] bit for bit.
    spec = W.CAUSAL_GQA_PREFILL
    q, k, v = W.make_prefill_spec(spec)
    o, l = gpu_fwd(q, k, v, True, W.fp32_scale(spec.D))
    G = spec.Hq // spec.Hkv
    v_rep = v.repeat_interleave(G, dim=1)
    assert torch.equal(o[:, :, 0].cpu(), v_rep[:, :, 0])


def test_identity_values_expose_probabilities():
    # V = I (kv_len <= D): O rows are the softmax rows P.
    Lq, Lk, D = 100, 128, 128
    q, k, _ = W.make_prefill(1, 4, 1, Lq, Lk, D, "bf16", seed=77)
    v = torch.eye(Lk, D).view(1, 1, Lk, D).to(torch.bfloat16)
    o, _ = gpu_fwd(q, k, v, True, W.fp32_scale(D))
    o = o.double().cpu().numpy()
    for h in range(4):
        p = oracle.softmax_matrix(q, k, W.fp32_scale(D), True, 0, h)
        assert np.abs(o[0, h] - p).max() <= 2e-2
        np.testing.assert_allclose(o[0, h].sum(axis=1), 1.0, atol=2e-2)


def test_deterministic():
    q, k, v = W.make_prefill(2, 8, 2, 300, 300, 128, "bf16", seed=3)
    o1, l1 = gpu_fwd(q, k, v, True, 0.1)
    o2, l2 = gpu_fwd(q, k, v, True, 0.1)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_large_scores_stable():
    q, k, v = W.make_prefill(1, 4, 2, 130, 130, 64, "bf16", seed=9)
    q = (q.float() * 30).to(torch.bfloat16)  # scores of order 100s
    scale = W.fp32_scale(64)
    o, l = gpu_fwd(q, k, v, True, scale)
    o_ref, l_ref = oracle.attn_fwd(q, k, v, scale, True)
    check(o.double().cpu().numpy(), l.double().cpu().numpy(), o_ref, l_ref, "bf16", "x30")


# ---- decode -----------------------------------------------------------------

def gpu_decode(inp, n_splits, scale, paged=True):
    q = inp.q.cuda()
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    if paged:
        o, l = gqa.attn_decode_splitk(q, inp.k_cache.cuda(), inp.v_cache.cuda(), inp.seq_lens.cuda(),
                                      block_table=inp.block_table.cuda(), n_splits=n_splits,
                                      scale=scale, max_kv_len=inp.max_kv_len, out=out, lse=lse)
    else:
        o, l = gqa.attn_decode_splitk(q, inp.k_dense.cuda(), inp.v_dense.cuda(), inp.seq_lens.cuda(),
                                      n_splits=n_splits, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), l.double().cpu().numpy()


def test_decode_workload_all_rows():
    spec = W.PAGED_DECODE
    print("workload paged_decode", flush=True)
    inp = W.make_decode_spec(spec)
    scale = W.fp32_scale(spec.D)
    o, l = gpu_decode(inp, spec.n_splits, scale)
    o_ref, l_ref = oracle.attn_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, scale,
                                      block_table=inp.block_table, max_kv_len=inp.max_kv_len)
    e_o, e_l = check(o, l, o_ref, l_ref, "bf16", "paged_decode")
    print(f"paged_decode: max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}")


DECODE = [
    # B, Hq, Hkv, D, dtype, len_lo, len_hi, page_size, n_splits
    (4, 32, 8, 128, "bf16", 1, 700, 256, 16),
    (3, 8, 8, 64, "f16", 1, 300, 16, 3),
    (2, 16, 2, 128, "bf16", 100, 2000, 64, 64),     # G = 8
    (5, 4, 2, 128, "f16", 1, 63, 1, 1),             # page size 1, one split
    (2, 6, 3, 64, "bf16", 500, 900, 128, 7),        # G = 2
    (2, 32, 1, 128, "bf16", 100, 1500, 32, 8),      # G = 32: two blocks of 16 heads
    (2, 20, 2, 64, "f16", 1, 400, 8, 5),            # G = 10, page size 8
    (3, 8, 2, 128, "bf16", 2000, 5000, 16, 256),    # many splits, page size 16
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "-".join(map(str, c)))
def test_decode_cases(case):
    B, Hq, Hkv, D, dt, lo, hi, ps, ns = case
    print(f"decode case {case}", flush=True)
    inp = W.make_decode(B, Hq, Hkv, D, dt, seed=sum(case[:4]) + hi, len_lo=lo, len_hi=hi, page_size=ps)
    scale = W.fp32_scale(D)
    o, l = gpu_decode(inp, ns, scale)
    o_ref, l_ref = oracle.attn_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, scale,
                                      block_table=inp.block_table, max_kv_len=inp.max_kv_len)
    check(o, l, o_ref, l_ref, dt, str(case))


# Chunks of more than 4096 keys: a wave's 16-token slices go round-robin over
# the 4 waves, so past its 64th slice a wave reads each slice's page id from the
# block table itself instead of from the per-lane list loaded with the chunk.
LONG_CHUNK = [
    # B, Hq, Hkv, D, dtype, len_lo, len_hi, page_size, n_splits
    (2, 8, 2, 128, "bf16", 9000, 20000, 256, 1),
    (2, 8, 2, 64, "f16", 9000, 20000, 16, 2),
]


@pytest.mark.parametrize("case", LONG_CHUNK, ids=lambda c: "-".join(map(str, c)))
def test_decode_long_chunks(case):
    B, Hq, Hkv, D, dt, lo, hi, ps, ns = case
    print(f"decode long chunks {case}", flush=True)
    inp = W.make_decode(B, Hq, Hkv, D, dt, seed=sum(case[:4]) + hi, len_lo=lo, len_hi=hi, page_size=ps)
    assert int(inp.seq_lens.min()) > 4096 * ns  # every chunk spans more than 64 slices per wave
    scale = W.fp32_scale(D)
    o, l = gpu_decode(inp, ns, scale)
    o_ref, l_ref = oracle.attn_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, scale,
                                      block_table=inp.block_table, max_kv_len=inp.max_kv_len)
    check(o, l, o_ref, l_ref, dt, str(case))


def test_decode_empty_and_short_sequences():
    inp = W.make_decode(4, 8, 2, 128, "bf16", seed=5, seq_lens=[0, 1, 64, 65], page_size=64, max_pages=2)
    inp.block_table[0, 0] = 0  # never read for an empty sequence
    o, l = gpu_decode(inp, 16, 0.09)
    o_ref, l_ref = oracle.attn_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, 0.09,
                                      block_table=inp.block_table, max_kv_len=inp.max_kv_len)
    check(o, l, o_ref, l_ref, "bf16", "empty/short")
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))


def test_decode_split_count_invariance():
    inp = W.make_decode(3, 16, 4, 128, "bf16", seed=6, len_lo=200, len_hi=3000, page_size=256)
    res = [gpu_decode(inp, ns, 0.088) for ns in (1, 2, 5, 16, 64)]
    o_ref, l_ref = oracle.attn_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, 0.088,
                                      block_table=inp.block_table, max_kv_len=inp.max_kv_len)
    for o, l in res:
        check(o, l, o_ref, l_ref, "bf16", "split invariance")


def test_decode_page_permutation_bitwise():
    kw = dict(B=3, Hq=8, Hkv=2, D=128, dtype="bf16", seed=8, len_lo=300, len_hi=900, page_size=64)
    a = W.make_decode(**kw, permute=True)
    b = W.make_decode(**kw, permute=False)
    ka = torch.empty_like(a.k_cache)
    va = torch.empty_like(a.v_cache)
    for s in range(3):
        n = (int(a.seq_lens[s]) + 63) // 64
        ka[a.block_table[s, :n].long()] = b.k_cache[b.block_table[s, :n].long()]
        va[a.block_table[s, :n].long()] = b.v_cache[b.block_table[s, :n].long()]
    a.k_cache, a.v_cache = ka, va
    o1, l1 = gpu_decode(a, 16, 0.1)
    o2, l2 = gpu_decode(b, 16, 0.1)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_decode_dense_matches_paged():
    inp = W.make_decode(3, 8, 2, 64, "f16", seed=10, len_lo=10, len_hi=500, page_size=32)
    L = inp.max_kv_len
    kd = torch.zeros(3, 2, L, 64, dtype=torch.float16)
    vd = torch.zeros(3, 2, L, 64, dtype=torch.float16)
    for s in range(3):
        n = int(inp.seq_lens[s])
        pages = inp.block_table[s, :(n + 31) // 32].long()
        kd[s, :, :n] = inp.k_cache[pages].reshape(-1, 2, 64)[:n].permute(1, 0, 2)
        vd[s, :, :n] = inp.v_cache[pages].reshape(-1, 2, 64)[:n].permute(1, 0, 2)
    inp.k_dense, inp.v_dense = kd, vd
    o1, l1 = gpu_decode(inp, 4, 0.125, paged=True)
    o2, l2 = gpu_decode(inp, 4, 0.125, paged=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o_ref, l_ref = oracle.attn_decode(inp.q, kd, vd, inp.seq_lens, 0.125)
    check(o2, l2, o_ref, l_ref, "f16", "dense")


# ---- several queries per sequence ---------------------------------------------

def gpu_decode_multi(inp, n_splits, scale, paged=True):
    q = inp.q.cuda()
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    if paged:
        o, l = gqa.attn_decode_splitk_multi(q, inp.k_cache.cuda(), inp.v_cache.cuda(), inp.seq_lens.cuda(),
                                            block_table=inp.block_table.cuda(), n_splits=n_splits,
                                            scale=scale, max_kv_len=inp.max_kv_len, out=out, lse=lse)
    else:
        o, l = gqa.attn_decode_splitk_multi(q, inp.k_dense.cuda(), inp.v_dense.cuda(), inp.seq_lens.cuda(),
                                            n_splits=n_splits, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), l.double().cpu().numpy()


def oracle_multi(inp, scale, k=None, v=None, block_table="pool"):
    if block_table == "pool":
        return oracle.attn_decode_multi(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, scale,
                                        block_table=inp.block_table, max_kv_len=inp.max_kv_len)
    return oracle.attn_decode_multi(inp.q, k, v, inp.seq_lens, scale)


def test_decode_multi_workload_all_rows():
    spec = W.MULTI_QUERY_DECODE
    print("workload multi_query_decode", flush=True)
    inp = W.make_decode_spec(spec)
    scale = W.fp32_scale(spec.D)
    o, l = gpu_decode_multi(inp, spec.n_splits, scale)
    o_ref, l_ref = oracle_multi(inp, scale)
    e_o, e_l = check(o, l, o_ref, l_ref, "bf16", "multi_query_decode")
    print(f"multi_query_decode: max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}")


DECODE_MULTI = [
    # B, Hq, Hkv, D, dtype, q_len, len_lo, len_hi, page_size, n_splits
    (4, 32, 8, 128, "bf16", 4, 1, 700, 256, 16),      # 4 heads x 4 queries: one block of 16 columns
    (3, 8, 2, 128, "f16", 2, 1, 300, 16, 3),
    (2, 16, 2, 128, "bf16", 8, 100, 2000, 64, 64),    # 8 heads x 8 queries: four column blocks
    (5, 4, 2, 64, "f16", 16, 1, 63, 1, 1),            # page size 1; some sequences shorter than q_len
    (2, 6, 3, 64, "bf16", 3, 500, 900, 128, 7),       # 6 columns
    (3, 32, 4, 128, "bf16", 5, 1, 200, 16, 16),       # 40 columns: a ragged last block; many empty splits
    (2, 8, 2, 128, "bf16", 256, 300, 900, 64, 8),     # q_len at its maximum: 1024 columns, 64 blocks
    (2, 4, 4, 64, "f16", 256, 1, 300, 16, 4),         # maximum q_len over sequences shorter than it
]


@pytest.mark.parametrize("case", DECODE_MULTI, ids=lambda c: "-".join(map(str, c)))
def test_decode_multi_cases(case):
    B, Hq, Hkv, D, dt, q_len, lo, hi, ps, ns = case
    print(f"multi-query decode case {case}", flush=True)
    inp = W.make_decode(B, Hq, Hkv, D, dt, seed=sum(case[:4]) + hi + q_len, len_lo=lo, len_hi=hi,
                        page_size=ps, q_len=q_len)
    scale = W.fp32_scale(D)
    o, l = gpu_decode_multi(inp, ns, scale)
    o_ref, l_ref = oracle_multi(inp, scale)
    check(o, l, o_ref, l_ref, dt, str(case))


def test_decode_multi_long_chunks():
    # one chunk of 9000-20000 keys per sequence: page ids past a wave's 64th
    # slice come from the block table directly
    print("decode multi long chunks", flush=True)
    inp = W.make_decode(2, 8, 2, 128, "bf16", seed=77, len_lo=9000, len_hi=20000, page_size=64, q_len=4)
    o, l = gpu_decode_multi(inp, 1, 0.088)
    o_ref, l_ref = oracle_multi(inp, 0.088)
    check(o, l, o_ref, l_ref, "bf16", "multi long chunks")


def test_decode_multi_short_sequences_and_invisible_chunks():
    # len 0: nothing; len 1 and 3 with 16 queries: the leading queries see no key;
    # len 961 with 16 splits: the last 64-token chunk holds key 960 only, which the
    # first 15 queries do not see, so that chunk weighs 0 for them.
    inp = W.make_decode(5, 8, 2, 128, "bf16", seed=31, seq_lens=[0, 1, 3, 961, 64], page_size=64,
                        max_pages=16, q_len=16)
    inp.block_table[0, 0] = 0  # never read for an empty sequence
    o, l = gpu_decode_multi(inp, 16, 0.09)
    o_ref, l_ref = oracle_multi(inp, 0.09)
    check(o, l, o_ref, l_ref, "bf16", "short / invisible chunks")
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    assert np.all(np.isneginf(l[1, :, :15])) and np.all(np.isfinite(l[1, :, 15]))


def test_decode_multi_single_query_equals_decode_bitwise():
    inp = W.make_decode(3, 16, 4, 128, "bf16", seed=32, len_lo=200, len_hi=3000, page_size=256)
    o1, l1 = gpu_decode(inp, 16, 0.088)
    inp.q = inp.q.unsqueeze(2).contiguous()
    o2, l2 = gpu_decode_multi(inp, 16, 0.088)
    assert np.array_equal(o1, o2[:, :, 0]) and np.array_equal(l1, l2[:, :, 0])


def test_decode_multi_dense_matches_paged():
    inp = W.make_decode(3, 8, 2, 64, "f16", seed=33, len_lo=1, len_hi=500, page_size=32, q_len=6)
    L = inp.max_kv_len
    kd = torch.zeros(3, 2, L, 64, dtype=torch.float16)
    vd = torch.zeros(3, 2, L, 64, dtype=torch.float16)
    for s in range(3):
        n = int(inp.seq_lens[s])
        pages = inp.block_table[s, :(n + 31) // 32].long()
        kd[s, :, :n] = inp.k_cache[pages].reshape(-1, 2, 64)[:n].permute(1, 0, 2)
        vd[s, :, :n] = inp.v_cache[pages].reshape(-1, 2, 64)[:n].permute(1, 0, 2)
    inp.k_dense, inp.v_dense = kd, vd
    o1, l1 = gpu_decode_multi(inp, 4, 0.125, paged=True)
    o2, l2 = gpu_decode_multi(inp, 4, 0.125, paged=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o_ref, l_ref = oracle_multi(inp, 0.125, kd, vd, block_table=None)
    check(o2, l2, o_ref, l_ref, "f16", "dense multi")


# ---- ragged prefill over a paged cache ------------------------------------------

def gpu_prefill_paged(inp, causal, scale, last=True, kernel=None):
    q = inp.q.cuda()
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    o, l = gqa.attn_prefill_paged(q, inp.k_cache.cuda(), inp.v_cache.cuda(), inp.qo_indptr.cuda(),
                                  inp.kv_indptr.cuda(), inp.kv_indices.cuda(), inp.max_q_len,
                                  kv_last_page_len=inp.kv_last_page_len.cuda() if last else None,
                                  causal=causal, scale=scale, out=out, lse=lse, kernel=kernel)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), l.double().cpu().numpy()


def oracle_prefill_paged(inp, causal, scale, rows=None, last=True):
    return oracle.attn_prefill_paged(inp.q, inp.k_cache, inp.v_cache, inp.qo_indptr, inp.kv_indptr,
                                     inp.kv_indices, scale, causal,
                                     inp.kv_last_page_len if last else None, rows=rows)


PAGED_PREFILL = [
    # Hq, Hkv, D, dtype, page_size, causal, (q_lens, kv_lens) or (B, q range, prefix range)
    (8, 2, 128, "bf16", 1, True, ([3, 0, 70, 129, 1], [9, 4, 0, 200, 300])),
    (4, 4, 64, "f16", 16, True, (5, (1, 300), (0, 300))),        # G = 1
    (32, 4, 128, "bf16", 64, True, (3, (1, 400), (0, 500))),      # G = 8
    (6, 3, 64, "bf16", 256, False, (4, (1, 200), (0, 300))),      # G = 2, non-causal
    (16, 2, 128, "f16", 4, True, ([200, 64, 7, 130], [150, 64, 3, 400])),  # some q_len > kv_len
    (8, 2, 128, "bf16", 16, True, (70, (1, 40), (0, 60))),       # > 64 requests (work order over 2 lane chunks)
    (4, 2, 64, "bf16", 16, True, (520, (1, 8), (0, 12))),        # > 512 requests: the dense work order
    (8, 2, 128, "bf16", 8, True, (300, (1, 70), (0, 900))),      # 5 chunks of requests, prefixes 0-900: long-first order
    (8, 4, 64, "f16", 32, False, (100, (1, 130), (0, 400))),     # non-causal over 2 chunks
]


# both kernels have a paged mode (chosen by the grid size; forced here)
@pytest.mark.parametrize("kernel", PREFILL_KERNELS)
@pytest.mark.parametrize("case", PAGED_PREFILL, ids=lambda c: "-".join(map(str, c[:6])))
def test_prefill_paged_cases(case, kernel):
    Hq, Hkv, D, dt, ps, causal, lens = case
    print(f"paged prefill case {case[:6]} kernel {kernel}", flush=True)
    if isinstance(lens[0], list):
        inp = W.make_paged_prefill(len(lens[0]), Hq, Hkv, D, dt, seed=Hq + D + ps, page_size=ps,
                                   q_lens=lens[0], kv_lens=lens[1])
    else:
        B, (qlo, qhi), (plo, phi) = lens
        inp = W.make_paged_prefill(B, Hq, Hkv, D, dt, seed=Hq + D + ps, q_lo=qlo, q_hi=qhi,
                                   prefix_lo=plo, prefix_hi=phi, page_size=ps)
    scale = W.fp32_scale(D)
    o, l = gpu_prefill_paged(inp, causal, scale, kernel=kernel)
    o_ref, l_ref = oracle_prefill_paged(inp, causal, scale)
    check(o, l, o_ref, l_ref, dt, str(case[:6]))


@pytest.mark.parametrize("kernel", PREFILL_KERNELS)
def test_prefill_paged_full_pages_without_last_len(kernel):
    # kv_last_page_len omitted: every page is full
    inp = W.make_paged_prefill(3, 8, 2, 64, "bf16", seed=50, page_size=32, q_lens=[40, 64, 3],
                               kv_lens=[64, 96, 32])
    o, l = gpu_prefill_paged(inp, True, 0.125, last=False, kernel=kernel)
    o_ref, l_ref = oracle_prefill_paged(inp, True, 0.125, last=False)
    check(o, l, o_ref, l_ref, "bf16", "full pages")


@pytest.mark.parametrize("kernel", PREFILL_KERNELS)
def test_prefill_paged_equals_dense_forward(kernel):
    # one request over an identity page table is the dense forward of the same
    # K/V on the same kernel
    inp = W.make_paged_prefill(1, 8, 2, 128, "bf16", seed=51, page_size=64, q_lens=[300], kv_lens=[700],
                               permute=False)
    o1, l1 = gpu_prefill_paged(inp, True, 0.088, kernel=kernel)
    kd = inp.k_cache.reshape(-1, 2, 128)[:700].permute(1, 0, 2).unsqueeze(0).contiguous()
    vd = inp.v_cache.reshape(-1, 2, 128)[:700].permute(1, 0, 2).unsqueeze(0).contiguous()
    qd = inp.q.permute(1, 0, 2).unsqueeze(0).contiguous()
    o2, l2 = gpu_fwd(qd, kd, vd, True, 0.088, kernel=kernel)
    o2 = o2.double().cpu().numpy()[0].transpose(1, 0, 2)
    l2 = l2.double().cpu().numpy()[0].T
    # the same kernel arithmetic on the same keys: bitwise equal
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


_RAGGED_ORACLE = {}


@pytest.mark.parametrize("kernel", PREFILL_KERNELS)
def test_prefill_paged_workload_all_elements(kernel):
    spec = W.RAGGED_PAGED_PREFILL
    print(f"workload ragged_paged_prefill kernel {kernel}", flush=True)
    if "ref" not in _RAGGED_ORACLE:
        inp = W.make_paged_prefill_spec(spec)
        scale = W.fp32_scale(spec.D)
        _RAGGED_ORACLE["ref"] = (inp, scale, oracle_prefill_paged(inp, spec.causal, scale))
    inp, scale, (o_ref, l_ref) = _RAGGED_ORACLE["ref"]
    o, l = gpu_prefill_paged(inp, spec.causal, scale, kernel=kernel)
    e_o, e_l = check(o, l, o_ref, l_ref, "bf16", "ragged_paged_prefill")
    print(f"ragged_paged_prefill ({kernel}): all {l_ref.size} rows, max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}")


# ---- decode over an 8-bit E4M3 cache ----------------------------------------------

def gpu_decode_fp8(inp, n_splits, scale, dense=None):
    q = inp.q.cuda()
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    if dense is None:
        o, l = gqa.attn_decode_splitk_fp8(q, inp.k8.cuda(), inp.v8.cuda(), inp.k_ss.cuda(), inp.v_ss.cuda(),
                                          inp.seq_lens.cuda(), block_table=inp.block_table.cuda(),
                                          n_splits=n_splits, scale=scale, max_kv_len=inp.max_kv_len,
                                          out=out, lse=lse)
    else:
        k8, v8, kss, vss = (t.cuda() for t in dense)
        o, l = gqa.attn_decode_splitk_fp8(q, k8, v8, kss, vss, inp.seq_lens.cuda(), n_splits=n_splits,
                                          scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), l.double().cpu().numpy()


def oracle_fp8(inp, scale, rows=None, dense=None):
    if dense is None:
        return oracle.attn_decode_fp8(inp.q, inp.k8, inp.v8, inp.k_ss, inp.v_ss, inp.seq_lens, scale,
                                      block_table=inp.block_table, max_kv_len=inp.max_kv_len, rows=rows)
    k8, v8, kss, vss = dense
    return oracle.attn_decode_fp8(inp.q, k8, v8, kss, vss, inp.seq_lens, scale, rows=rows)


def test_decode_fp8_workload_all_rows():
    spec = W.FP8_PAGED_DECODE
    print("workload fp8_paged_decode", flush=True)
    inp = W.make_decode_fp8_spec(spec)
    scale = W.fp32_scale(spec.D)
    o, l = gpu_decode_fp8(inp, spec.n_splits, scale)
    o_ref, l_ref = oracle_fp8(inp, scale)
    e_o, e_l = check(o, l, o_ref, l_ref, "bf16", "fp8_paged_decode")
    print(f"fp8_paged_decode: max|dO|={e_o:.3e} max|dLSE|={e_l:.3e}")


DECODE_FP8 = [
    # B, Hq, Hkv, D, dtype, len_lo, len_hi, page_size, n_splits
    (4, 32, 8, 128, "bf16", 1, 700, 256, 16),
    (3, 8, 8, 64, "f16", 1, 300, 16, 3),            # G = 1, 16-token pages
    (2, 16, 2, 128, "bf16", 100, 2000, 64, 64),     # G = 8
    (2, 6, 3, 64, "bf16", 500, 900, 128, 7),        # G = 2
    (2, 32, 1, 128, "bf16", 100, 1500, 32, 8),      # G = 32: two blocks of 16 heads
    (2, 20, 2, 64, "f16", 1, 400, 16, 5),           # G = 10
]


@pytest.mark.parametrize("case", DECODE_FP8, ids=lambda c: "-".join(map(str, c)))
def test_decode_fp8_cases(case):
    B, Hq, Hkv, D, dt, lo, hi, ps, ns = case
    print(f"fp8 decode case {case}", flush=True)
    inp = W.make_decode_fp8(B, Hq, Hkv, D, dt, seed=sum(case[:4]) + hi + 7, len_lo=lo, len_hi=hi, page_size=ps)
    scale = W.fp32_scale(D)
    o, l = gpu_decode_fp8(inp, ns, scale)
    o_ref, l_ref = oracle_fp8(inp, scale)
    check(o, l, o_ref, l_ref, dt, str(case))


def test_decode_fp8_long_chunks():
    # one chunk of 9000-20000 keys per sequence (more than 64 slices per wave)
    print("fp8 decode long chunks", flush=True)
    inp = W.make_decode_fp8(2, 8, 2, 128, "bf16", seed=78, len_lo=9000, len_hi=20000, page_size=256)
    o, l = gpu_decode_fp8(inp, 1, 0.088)
    o_ref, l_ref = oracle_fp8(inp, 0.088)
    check(o, l, o_ref, l_ref, "bf16", "fp8 long chunks")


def test_decode_fp8_empty_and_short_sequences():
    inp = W.make_decode_fp8(4, 8, 2, 128, "bf16", seed=70, seq_lens=[0, 1, 64, 65], page_size=64, max_pages=2)
    inp.block_table[0, 0] = 0  # never read for an empty sequence
    o, l = gpu_decode_fp8(inp, 16, 0.09)
    o_ref, l_ref = oracle_fp8(inp, 0.09)
    check(o, l, o_ref, l_ref, "bf16", "fp8 empty/short")
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))


def _fp8_dense(inp, Hkv, D):
    B = inp.q.shape[0]
    L = inp.max_kv_len
    ps = inp.page_size
    k8 = torch.zeros(B, Hkv, L, D, dtype=torch.uint8)
    v8 = torch.zeros(B, Hkv, L, D, dtype=torch.uint8)
    kss = torch.zeros(B, Hkv, L, dtype=torch.int32)
    vss = torch.zeros(B, Hkv, L, dtype=torch.int32)
    for b in range(B):
        n = int(inp.seq_lens[b])
        pages = inp.block_table[b, :(n + ps - 1) // ps].long()
        k8[b, :, :n] = inp.k8[pages].reshape(-1, Hkv, D)[:n].permute(1, 0, 2)
        v8[b, :, :n] = inp.v8[pages].reshape(-1, Hkv, D)[:n].permute(1, 0, 2)
        kss[b, :, :n] = inp.k_ss[pages].reshape(-1, Hkv)[:n].permute(1, 0)
        vss[b, :, :n] = inp.v_ss[pages].reshape(-1, Hkv)[:n].permute(1, 0)
    return k8, v8, kss, vss


def test_decode_fp8_dense_matches_paged_and_page_order():
    kw = dict(B=3, Hq=8, Hkv=2, D=64, dtype="f16", seed=71, len_lo=10, len_hi=500, page_size=32)
    a = W.make_decode_fp8(**kw, permute=True)
    o1, l1 = gpu_decode_fp8(a, 4, 0.125)
    dense = _fp8_dense(a, 2, 64)
    o2, l2 = gpu_decode_fp8(a, 4, 0.125, dense=dense)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o_ref, l_ref = oracle_fp8(a, 0.125, dense=dense)
    check(o2, l2, o_ref, l_ref, "f16", "fp8 dense")
    # the same logical cache with its pages in reverse order in the pool
    n_pool = a.k8.shape[0]
    b = W.DecodeFp8Inputs(a.q, a.k8.flip(0).contiguous(), a.v8.flip(0).contiguous(),
                          a.k_ss.flip(0).contiguous(), a.v_ss.flip(0).contiguous(), a.seq_lens,
                          torch.where(a.block_table >= 0, n_pool - 1 - a.block_table, a.block_table),
                          a.page_size, a.max_kv_len)
    o3, l3 = gpu_decode_fp8(b, 4, 0.125)
    assert np.array_equal(o1, o3) and np.array_equal(l1, l3)


# ---- operands past 2^31 elements: every offset is 64-bit ---------------------------
# Each case puts the data it checks where element offsets are >= 2^31 (byte
# offsets >= 4 GiB) and fills everything else with NaN: an offset that wrapped
# at 32 bits would read NaN (or write the wrong rows) and fail the comparison.
# The GPU result must also equal, bit for bit, the same call on a compact copy.

BIG = 2 ** 31
NAN_E4M3 = 0x7F                 # E4M3 byte with every exponent and mantissa bit set: NaN
NAN_SCALE_SHIFT = 0x7E007E00    # fp16 NaN in both halves of a scale-shift word


def _release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _pool(small, first, fill):
    """`small` (pages on the host) at page ids first.. of a pool on the GPU whose
    other pages hold `fill`."""
    pool = torch.full((first + small.shape[0],) + tuple(small.shape[1:]), fill, dtype=small.dtype, device="cuda")
    pool[first:] = small.cuda()
    return pool


def _shift_table(t, first):
    return torch.where(t >= 0, t + first, t)


def _last_batch(shape, data):
    """A NaN tensor of `shape` on the GPU whose last batch entry is `data` [1, ...]."""
    x = torch.full(shape, float("nan"), dtype=data.dtype, device="cuda")
    x[shape[0] - 1] = data[0].cuda()
    return x


@pytest.mark.parametrize("kernel", PREFILL_KERNELS + ["split", "f32"])
def test_prefill_kv_past_2g_elements(kernel):
    # 129 sequences of 65536 keys: the last sequence's K and V start at element 2^31
    dt = "f32" if kernel == "f32" else "bf16"
    B, Hq, Hkv, ql, kl, D = (129, 2, 2, 64, 65536, 128) if dt == "f32" else (129, 8, 2, 64, 65536, 128)
    assert (B - 1) * Hkv * kl * D == BIG
    kern = kernel if kernel in PREFILL_KERNELS else None
    splits = 2 if kernel == "split" else 1
    print(f"prefill K/V past 2^31 elements, kernel {kernel}", flush=True)
    q1, k1, v1 = W.make_prefill(1, Hq, Hkv, ql, kl, D, dt, seed=131)
    scale = W.fp32_scale(D)
    q = _last_batch((B, Hq, ql, D), q1)
    k = _last_batch((B, Hkv, kl, D), k1)
    v = _last_batch((B, Hkv, kl, D), v1)
    o, l = gqa.attn_fwd(q, k, v, causal=True, scale=scale, kv_splits=splits, kernel=kern)
    o_big, l_big = o[B - 1:].cpu(), l[B - 1:].cpu()
    del q, k, v, o, l
    _release()
    o_small, l_small = gqa.attn_fwd(q1.cuda(), k1.cuda(), v1.cuda(), causal=True, scale=scale, kv_splits=splits,
                                    kernel=kern)
    assert torch.equal(o_big, o_small.cpu()) and torch.equal(l_big, l_small.cpu())
    o_ref, l_ref = oracle.attn_fwd(q1, k1, v1, scale, True)
    check(o_big.double().numpy(), l_big.double().numpy(), o_ref, l_ref, dt, f"K/V past 2^31, {kernel}")


@pytest.mark.parametrize("kernel", PREFILL_KERNELS)
def test_prefill_qo_past_2g_elements(kernel):
    # 1025 sequences x 8 heads x 2048 positions x 128 dims: the last sequence's
    # Q and O rows start at element 2^31
    B, Hq, Hkv, L, D = 1025, 8, 2, 2048, 128
    assert (B - 1) * Hq * L * D == BIG
    print(f"prefill Q/O past 2^31 elements, kernel {kernel}", flush=True)
    q1, k1, v1 = W.make_prefill(1, Hq, Hkv, L, L, D, "bf16", seed=1025)
    scale = W.fp32_scale(D)
    q = _last_batch((B, Hq, L, D), q1)
    k = _last_batch((B, Hkv, L, D), k1)
    v = _last_batch((B, Hkv, L, D), v1)
    o, l = gqa.attn_fwd(q, k, v, causal=True, scale=scale, kv_splits=1, kernel=kernel)
    o_big, l_big = o[B - 1:].cpu(), l[B - 1:].cpu()
    del q, k, v, o, l
    _release()
    o_small, l_small = gqa.attn_fwd(q1.cuda(), k1.cuda(), v1.cuda(), causal=True, scale=scale, kv_splits=1,
                                    kernel=kernel)
    assert torch.equal(o_big, o_small.cpu()) and torch.equal(l_big, l_small.cpu())
    o_ref, l_ref = oracle.attn_fwd(q1, k1, v1, scale, True)
    check(o_big.double().numpy(), l_big.double().numpy(), o_ref, l_ref, "bf16", f"Q/O past 2^31, {kernel}")


def test_decode_pages_past_4gib():
    # 256-token pages of 8 heads x 128 dims (512 KiB): page 8192 starts at element
    # 2^31; every page the block table names sits at or above it
    B, Hq, Hkv, D, ps, first = 4, 32, 8, 128, 256, 8192
    assert first * ps * Hkv * D == BIG
    scale = W.fp32_scale(D)
    for q_len in (None, 4):
        print(f"decode pages past 4 GiB, q_len {q_len}", flush=True)
        inp = W.make_decode(B, Hq, Hkv, D, "bf16", seed=4096 + (q_len or 1), len_lo=300, len_hi=3000,
                            page_size=ps, q_len=q_len)
        big = W.DecodeInputs(inp.q, _pool(inp.k_cache, first, float("nan")), _pool(inp.v_cache, first, float("nan")),
                             inp.seq_lens, _shift_table(inp.block_table, first), ps, inp.max_kv_len)
        run = gpu_decode if q_len is None else gpu_decode_multi
        o_big, l_big = run(big, 16, scale)
        del big
        _release()
        o_small, l_small = run(inp, 16, scale)
        assert np.array_equal(o_big, o_small) and np.array_equal(l_big, l_small)
        if q_len is None:
            o_ref, l_ref = oracle.attn_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, scale,
                                              block_table=inp.block_table, max_kv_len=inp.max_kv_len)
        else:
            o_ref, l_ref = oracle_multi(inp, scale)
        check(o_big, l_big, o_ref, l_ref, "bf16", f"decode past 4 GiB, q_len {q_len}")


def test_decode_fp8_pages_past_4gib():
    # E4M3 pages of 256 tokens x 8 heads x 128 bytes (256 KiB): page 16384 starts
    # at byte 2^32
    B, Hq, Hkv, D, ps, first = 4, 32, 8, 128, 256, 16384
    assert first * ps * Hkv * D == 2 * BIG
    print("fp8 decode pages past 4 GiB", flush=True)
    inp = W.make_decode_fp8(B, Hq, Hkv, D, "bf16", seed=16384, len_lo=300, len_hi=3000, page_size=ps)
    scale = W.fp32_scale(D)
    big = W.DecodeFp8Inputs(inp.q, _pool(inp.k8, first, NAN_E4M3), _pool(inp.v8, first, NAN_E4M3),
                            _pool(inp.k_ss, first, NAN_SCALE_SHIFT), _pool(inp.v_ss, first, NAN_SCALE_SHIFT),
                            inp.seq_lens, _shift_table(inp.block_table, first), ps, inp.max_kv_len)
    o_big, l_big = gpu_decode_fp8(big, 16, scale)
    del big
    _release()
    o_small, l_small = gpu_decode_fp8(inp, 16, scale)
    assert np.array_equal(o_big, o_small) and np.array_equal(l_big, l_small)
    o_ref, l_ref = oracle_fp8(inp, scale)
    check(o_big, l_big, o_ref, l_ref, "bf16", "fp8 decode past 4 GiB")


@pytest.mark.parametrize("kernel", PREFILL_KERNELS)
def test_prefill_paged_pages_past_4gib(kernel):
    # paged prefill over 256-token pages of 8 heads x 128 dims: every page of
    # the batch at or above page 8192 (element 2^31)
    Hq, Hkv, D, ps, first = 32, 8, 128, 256, 8192
    print(f"paged prefill pages past 4 GiB, kernel {kernel}", flush=True)
    inp = W.make_paged_prefill(3, Hq, Hkv, D, "bf16", seed=8192, q_lo=1, q_hi=300, prefix_lo=0, prefix_hi=700,
                               page_size=ps)
    scale = W.fp32_scale(D)
    big = W.PagedPrefillInputs(inp.q, _pool(inp.k_cache, first, float("nan")),
                               _pool(inp.v_cache, first, float("nan")), inp.qo_indptr, inp.kv_indptr,
                               _shift_table(inp.kv_indices, first), inp.kv_last_page_len, ps, inp.max_q_len)
    o_big, l_big = gpu_prefill_paged(big, True, scale, kernel=kernel)
    del big
    _release()
    o_small, l_small = gpu_prefill_paged(inp, True, scale, kernel=kernel)
    assert np.array_equal(o_big, o_small) and np.array_equal(l_big, l_small)
    o_ref, l_ref = oracle_prefill_paged(inp, True, scale)
    check(o_big, l_big, o_ref, l_ref, "bf16", f"paged prefill past 4 GiB, {kernel}")
