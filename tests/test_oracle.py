"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against an independent route to the same number:
torch's own fp64 softmax / matmul / scaled_dot_product_attention on tiny
inputs, closed forms (uniform attention when K = 0, constant V, causal row 0,
the two-key logistic form), hand-derived golden fixtures, and invariants that
the definition fixes (key permutation, linearity in V, GQA = MHA with repeated
K/V heads, shift of all scores, paged = dense, split-merge = unsplit).
"""
import math
from fractions import Fraction
import json
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import make_prefill, make_decode, make_paged_prefill, make_decode_fp8, fp32_scale

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def torch_reference(q, k, v, scale, causal):
    """softmax(scale * Q K^T + mask) V in torch fp64 with an explicit bottom-right mask."""
    q, k, v = (t.to(torch.float64) for t in (q, k, v))
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    s = scale * torch.matmul(q, k.transpose(-1, -2).contiguous())
    if causal:
        i = torch.arange(Lq).view(-1, 1)
        j = torch.arange(Lk).view(1, -1)
        visible = j <= i + (Lk - Lq)
        s = s.masked_fill(~visible, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    row_empty = torch.isinf(lse) & (lse < 0)
    p = torch.softmax(s, dim=-1)
    p = torch.where(row_empty[..., None], torch.zeros_like(p), p)
    o = torch.matmul(p, v)
    return o.numpy(), lse.numpy()


SHAPES = [
    # B, Hq, Hkv, q_len, kv_len, D, causal
    (1, 1, 1, 1, 1, 4, True),
    (1, 2, 1, 5, 5, 8, True),
    (2, 4, 2, 7, 7, 16, False),
    (1, 4, 2, 6, 11, 8, True),     # q_len < kv_len: bottom-right offset
    (2, 8, 2, 9, 4, 8, True),      # q_len > kv_len: leading rows see nothing
    (1, 6, 3, 3, 13, 32, False),
    (1, 4, 1, 17, 33, 64, True),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_matches_torch_softmax(shape, dtype):
    B, Hq, Hkv, Lq, Lk, D, causal = shape
    q, k, v = make_prefill(B, Hq, Hkv, Lq, Lk, D, dtype, seed=hash(shape) % 1000)
    scale = fp32_scale(D)
    o, lse = oracle.attn_fwd(q, k, v, scale, causal)
    o_ref, lse_ref = torch_reference(q, k, v, scale, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=TOL)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=0, atol=TOL)
    assert np.all(lse[~fin] == -np.inf)


@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_sdpa(causal):
    # torch's SDPA aligns the causal mask top-left; with q_len == kv_len that
    # coincides with bottom-right, so it is an independent check there.
    q, k, v = make_prefill(2, 8, 2, 24, 24, 16, "f32", seed=5)
    scale = fp32_scale(16)
    o, _ = oracle.attn_fwd(q, k, v, scale, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.double(), k.double(), v.double(), is_causal=causal, scale=scale, enable_gqa=True)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=TOL)


@pytest.mark.parametrize("Lq,Lk", [(8, 8), (5, 12), (12, 5), (1, 9)])
def test_zero_keys_give_uniform_attention(Lq, Lk):
    # K = 0 makes every visible score 0: P is uniform over the visible keys, so
    # O[i] is the mean of the visible V rows and L_i = ln(count_i) with
    # count_i = min(kv_len, i + 1 + kv_len - q_len).  This pins the mask count.
    B, Hq, Hkv, D = 1, 4, 2, 8
    q, _, v = make_prefill(B, Hq, Hkv, Lq, Lk, D, "f32", seed=11)
    k = torch.zeros(B, Hkv, Lk, D, dtype=torch.float32)
    o, lse = oracle.attn_fwd(q, k, v, 0.3, True)
    vv = v.double().numpy()
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for i in range(Lq):
            n = max(0, min(Lk, i + 1 + Lk - Lq))
            if n == 0:
                assert lse[0, h, i] == -np.inf
                assert np.all(o[0, h, i] == 0)
                continue
            np.testing.assert_allclose(o[0, h, i], vv[0, g, :n].mean(axis=0), atol=TOL, rtol=0)
            assert abs(lse[0, h, i] - math.log(n)) < TOL


def test_constant_values():
    q, k, _ = make_prefill(1, 2, 1, 9, 9, 8, "f32", seed=3)
    v = torch.full((1, 1, 9, 8), 1.75)
    o, _ = oracle.attn_fwd(q, k, v, 0.5, True)
    np.testing.assert_allclose(o, 1.75, atol=TOL, rtol=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_causal_row_zero(dtype):
    # With delta = 0, row 0 sees only key 0: O[0] = V[0] exactly and
    # L_0 = scale * q_0 . k_0.
    q, k, v = make_prefill(1, 4, 2, 16, 16, 32, dtype, seed=7)
    scale = 0.125
    o, lse = oracle.attn_fwd(q, k, v, scale, True)
    for h in range(4):
        g = h // 2
        assert np.array_equal(o[0, h, 0], v[0, g, 0].double().numpy())
        dot = math.fsum(float(a) * float(b) for a, b in zip(q[0, h, 0].double(), k[0, g, 0].double()))
        assert abs(lse[0, h, 0] - scale * dot) < TOL


def test_two_keys_logistic_form():
    # Two visible keys: O = sigma(s0 - s1) v0 + sigma(s1 - s0) v1, L = logaddexp(s0, s1).
    q, k, v = make_prefill(1, 1, 1, 3, 2, 8, "f32", seed=21)
    scale = 0.7
    o, lse = oracle.attn_fwd(q, k, v, scale, False)
    qq, kk, vv = q.double().numpy()[0, 0], k.double().numpy()[0, 0], v.double().numpy()[0, 0]
    for i in range(3):
        s0 = scale * math.fsum(qq[i] * kk[0])
        s1 = scale * math.fsum(qq[i] * kk[1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        np.testing.assert_allclose(o[0, 0, i], w0 * vv[0] + (1 - w0) * vv[1], atol=TOL, rtol=0)
        assert abs(lse[0, 0, i] - np.logaddexp(s0, s1)) < TOL


def test_key_permutation_invariance():
    # Non-causal attention is a function of the set of (key, value) pairs.
    q, k, v = make_prefill(1, 4, 2, 6, 10, 16, "f32", seed=4)
    perm = torch.randperm(10, generator=torch.Generator().manual_seed(0))
    o1, l1 = oracle.attn_fwd(q, k, v, 0.25, False)
    o2, l2 = oracle.attn_fwd(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), 0.25, False)
    np.testing.assert_allclose(o1, o2, atol=TOL, rtol=0)
    np.testing.assert_allclose(l1, l2, atol=TOL, rtol=0)


def test_linear_in_values():
    q, k, v1 = make_prefill(1, 2, 2, 7, 7, 8, "f32", seed=8)
    v2 = torch.randn(v1.shape, generator=torch.Generator().manual_seed(9), dtype=torch.float64)
    v1 = v1.double()
    o1, _ = oracle.attn_fwd(q.double(), k.double(), v1, 0.3, True)
    o2, _ = oracle.attn_fwd(q.double(), k.double(), v2, 0.3, True)
    o12, _ = oracle.attn_fwd(q.double(), k.double(), v1 + 2.0 * v2, 0.3, True)
    np.testing.assert_allclose(o12, o1 + 2.0 * o2, atol=1e-11, rtol=0)


def test_gqa_equals_mha_with_repeated_heads():
    q, k, v = make_prefill(2, 8, 2, 9, 13, 16, "bf16", seed=10)
    o, l = oracle.attn_fwd(q, k, v, 0.2, True)
    o2, l2 = oracle.attn_fwd(q, k.repeat_interleave(4, dim=1), v.repeat_interleave(4, dim=1), 0.2, True)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_score_shift():
    # Adding c to every score leaves O unchanged and adds c to L.  The shift is
    # applied through one extra feature (q' = [q, 1], k' = [k, c / scale]);
    # c = 2000 would overflow exp() without the max subtraction.
    q, k, v = make_prefill(1, 2, 1, 5, 8, 8, "f32", seed=12)
    q, k, v = q.double(), k.double(), v.double()
    scale, c = 0.5, 2000.0
    o1, l1 = oracle.attn_fwd(q, k, v, scale, True)
    q2 = torch.cat([q, torch.ones(1, 2, 5, 1, dtype=torch.float64)], dim=-1)
    k2 = torch.cat([k, torch.full((1, 1, 8, 1), c / scale, dtype=torch.float64)], dim=-1)
    v2 = torch.cat([v, torch.zeros(1, 1, 8, 1, dtype=torch.float64)], dim=-1)
    o2, l2 = oracle.attn_fwd(q2, k2, v2, scale, True)
    np.testing.assert_allclose(o2[..., :8], o1, atol=1e-11, rtol=0)
    np.testing.assert_allclose(l2, l1 + c, atol=1e-9, rtol=0)


def test_softmax_matrix_rows_and_identity_values():
    # Rows of P sum to 1; with V = I the output rows are the rows of P.
    Lq, Lk, D = 6, 8, 8
    q, k, _ = make_prefill(1, 2, 1, Lq, Lk, D, "f32", seed=13)
    v = torch.eye(Lk, D).view(1, 1, Lk, D)
    p = oracle.softmax_matrix(q, k, 0.4, True, 0, 1)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=TOL, rtol=0)
    o, _ = oracle.attn_fwd(q, k, v, 0.4, True)
    np.testing.assert_allclose(o[0, 1], p, atol=TOL, rtol=0)
    s = 0.4 * (q[0, 1].double() @ k[0, 0].double().T)
    mask = torch.arange(Lk)[None, :] <= torch.arange(Lq)[:, None] + (Lk - Lq)
    ref = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=-1).numpy()
    np.testing.assert_allclose(p, ref, atol=TOL, rtol=0)


def test_row_subset_matches_full():
    q, k, v = make_prefill(2, 4, 2, 10, 14, 16, "bf16", seed=14)
    o, l = oracle.attn_fwd(q, k, v, 0.3, True)
    rows = np.array([0, 5, 17, 39, 79])
    o_r, l_r = oracle.attn_fwd(q, k, v, 0.3, True, rows=rows)
    np.testing.assert_array_equal(o_r, o.reshape(-1, 16)[rows])
    np.testing.assert_array_equal(l_r, l.reshape(-1)[rows])


# ---- storage-format widening ---------------------------------------------

def test_widen_every_f16_pattern():
    bits = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16)
    h = bits.view(torch.float16)
    got = oracle.widen(h)
    ref = h.numpy().astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_widen_every_bf16_pattern():
    bits = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16)
    b = bits.view(torch.bfloat16)
    got = oracle.widen(b)
    ref = b.to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


# ---- hand-derived golden fixtures -----------------------------------------

def _golden_cases():
    with open(os.path.join(GOLDEN, "closed_form_attention.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_closed_forms(case):
    q = torch.tensor(case["q"], dtype=torch.float64)
    k = torch.tensor([[math.log(float(Fraction(w))) for w in row] for row in case["k_log_of"]],
                     dtype=torch.float64)
    v = torch.tensor(case["v"], dtype=torch.float64)
    Hq, Lq, D = q.shape
    Hkv, Lk = k.shape
    q = q.view(1, Hq, Lq, D)
    k = k.view(1, Hkv, Lk, 1).expand(1, Hkv, Lk, D).contiguous() if D == 1 else None
    v = v.view(1, Hkv, Lk, -1)
    o, lse = oracle.attn_fwd(q, k, v, case["scale"], case["causal"])
    for h in range(Hq):
        for i in range(Lq):
            exp_o = [float(Fraction(x)) for x in case["expected_o"][h][i]]
            np.testing.assert_allclose(o[0, h, i], exp_o, atol=1e-14, rtol=0)
            e = case["expected_lse_log_of"][h][i]
            if e is None:
                assert lse[0, h, i] == -np.inf
            else:
                assert abs(lse[0, h, i] - math.log(float(Fraction(e)))) < 1e-14


# ---- decode ----------------------------------------------------------------

def test_decode_equals_prefill_single_query():
    # Decode of a sequence of length n is prefill with q_len = 1 over n keys;
    # with q_len = 1 the bottom-right causal mask shows every key.
    inp = make_decode(3, 8, 2, 16, "f32", seed=15, len_lo=5, len_hi=40, page_size=8)
    scale = 0.25
    o, l = oracle.attn_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, scale,
                              block_table=inp.block_table)
    for b in range(3):
        n = int(inp.seq_lens[b])
        pages = inp.block_table[b, :(n + 7) // 8].long()
        kd = inp.k_cache[pages].reshape(-1, 2, 16)[:n].permute(1, 0, 2).unsqueeze(0).contiguous()
        vd = inp.v_cache[pages].reshape(-1, 2, 16)[:n].permute(1, 0, 2).unsqueeze(0).contiguous()
        qd = inp.q[b].view(1, 8, 1, 16)
        o_ref, l_ref = torch_reference(qd, kd, vd, scale, True)
        np.testing.assert_allclose(o[b], o_ref[0, :, 0], atol=TOL, rtol=0)
        np.testing.assert_allclose(l[b], l_ref[0, :, 0], atol=TOL, rtol=0)


def test_paged_equals_dense_and_permutation_invariant():
    kw = dict(B=4, Hq=8, Hkv=4, D=32, dtype="bf16", seed=16, len_lo=1, len_hi=70, page_size=16)
    a = make_decode(**kw, permute=True)
    b = make_decode(**kw, permute=False)
    assert torch.equal(a.seq_lens, b.seq_lens)
    # the same logical K/V in both pools, placed differently
    k_log = b.k_cache.clone()
    v_log = b.v_cache.clone()
    ka = torch.empty_like(a.k_cache)
    va = torch.empty_like(a.v_cache)
    for bb in range(4):
        n = (int(a.seq_lens[bb]) + 15) // 16
        ka[a.block_table[bb, :n].long()] = k_log[b.block_table[bb, :n].long()]
        va[a.block_table[bb, :n].long()] = v_log[b.block_table[bb, :n].long()]
    o1, l1 = oracle.attn_decode(a.q, ka, va, a.seq_lens, 0.2, block_table=a.block_table)
    o2, l2 = oracle.attn_decode(b.q, k_log, v_log, b.seq_lens, 0.2, block_table=b.block_table)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # identity table over a dense [B, Hkv, L, D] copy
    L = int(b.seq_lens.max())
    kd = torch.zeros(4, 4, L, 32, dtype=torch.bfloat16)
    vd = torch.zeros(4, 4, L, 32, dtype=torch.bfloat16)
    for bb in range(4):
        n = int(b.seq_lens[bb])
        pages = b.block_table[bb, :(n + 15) // 16].long()
        kd[bb, :, :n] = k_log[pages].reshape(-1, 4, 32)[:n].permute(1, 0, 2)
        vd[bb, :, :n] = v_log[pages].reshape(-1, 4, 32)[:n].permute(1, 0, 2)
    o3, l3 = oracle.attn_decode(b.q, kd, vd, b.seq_lens, 0.2)
    assert np.array_equal(o2, o3) and np.array_equal(l2, l3)


def test_decode_empty_sequence():
    inp = make_decode(2, 4, 2, 16, "f32", seed=17, seq_lens=[0, 9], page_size=8, max_pages=2)
    inp.block_table[0, 0] = 0  # a table entry for an empty sequence is never read
    o, l = oracle.attn_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, 0.3,
                              block_table=inp.block_table)
    assert np.all(o[0] == 0) and np.all(l[0] == -np.inf)
    assert np.all(np.isfinite(l[1]))


@pytest.mark.parametrize("n_splits", [1, 2, 3, 16])
def test_split_merge_equals_unsplit(n_splits):
    inp = make_decode(3, 8, 2, 32, "bf16", seed=18, len_lo=1, len_hi=200, page_size=64)
    g = torch.Generator().manual_seed(n_splits)
    bounds = []
    for b in range(3):
        n = int(inp.seq_lens[b])
        # arbitrary monotone edges, some chunks empty and some past the end
        cuts = sorted(torch.randint(0, n + 40, (n_splits - 1,), generator=g).tolist())
        bounds.append([0] + cuts + [n + 40])
    o, l, op, lp = oracle.decode_split_merge(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, 0.125,
                                             bounds, block_table=inp.block_table)
    o_ref, l_ref = oracle.attn_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, 0.125,
                                      block_table=inp.block_table)
    np.testing.assert_allclose(o, o_ref.reshape(-1, 32), atol=TOL, rtol=0)
    np.testing.assert_allclose(l, l_ref.reshape(-1), atol=TOL, rtol=0)
    # empty chunks carry (0, -inf)
    for r in range(o.shape[0]):
        b = r // 8
        for s in range(n_splits):
            lo, hi = bounds[b][s], min(bounds[b][s + 1], int(inp.seq_lens[b]))
            if hi <= lo:
                assert lp[r, s] == -np.inf and np.all(op[r, s] == 0)
            else:
                assert np.isfinite(lp[r, s])


def test_split_merge_all_empty():
    inp = make_decode(1, 2, 1, 8, "f32", seed=19, seq_lens=[0], page_size=8, max_pages=1)
    o, l, _, _ = oracle.decode_split_merge(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, 0.3,
                                           [[0, 4, 8]], block_table=inp.block_table)
    assert np.all(o == 0) and np.all(l == -np.inf)


# ---- several queries per sequence ---------------------------------------------

def test_decode_multi_query_i_is_decode_of_a_prefix():
    # Query i sits at position len - q_len + i, so it is plain decode over the
    # first len - q_len + 1 + i keys (none if that is <= 0).
    q_len = 5
    inp = make_decode(3, 8, 2, 16, "f32", seed=22, len_lo=2, len_hi=40, page_size=8, q_len=q_len)
    o, l = oracle.attn_decode_multi(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, 0.3,
                                    block_table=inp.block_table)
    for i in range(q_len):
        lens_i = torch.clamp(inp.seq_lens - (q_len - 1 - i), min=0).to(torch.int32)
        oi, li = oracle.attn_decode(inp.q[:, :, i].contiguous(), inp.k_cache, inp.v_cache, lens_i, 0.3,
                                    block_table=inp.block_table)
        assert np.array_equal(o[:, :, i], oi) and np.array_equal(l[:, :, i], li)


@pytest.mark.parametrize("q_len,dtype", [(1, "f32"), (6, "f32"), (3, "bf16")])
def test_decode_multi_matches_torch_reference(q_len, dtype):
    # Against torch fp64 with an explicit bottom-right mask over a dense copy of
    # each sequence's keys, gathered here from the pool; sequences shorter than
    # q_len leave their leading queries with no visible key (o = 0, lse = -inf).
    inp = make_decode(4, 8, 2, 16, dtype, seed=23 + q_len, len_lo=1, len_hi=40, page_size=8, q_len=q_len)
    scale = 0.25
    o, l = oracle.attn_decode_multi(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, scale,
                                    block_table=inp.block_table)
    for b in range(4):
        n = int(inp.seq_lens[b])
        pages = inp.block_table[b, :(n + 7) // 8].long()
        kd = inp.k_cache[pages].reshape(-1, 2, 16)[:n].permute(1, 0, 2).unsqueeze(0).contiguous()
        vd = inp.v_cache[pages].reshape(-1, 2, 16)[:n].permute(1, 0, 2).unsqueeze(0).contiguous()
        o_ref, l_ref = torch_reference(inp.q[b:b + 1], kd, vd, scale, True)
        np.testing.assert_allclose(o[b], o_ref[0], atol=TOL, rtol=0)
        np.testing.assert_array_equal(np.isinf(l[b]), np.isinf(l_ref[0]))
        fin = np.isfinite(l_ref[0])
        np.testing.assert_allclose(l[b][fin], l_ref[0][fin], atol=TOL, rtol=0)


# ---- ragged prefill over a paged cache ---------------------------------------

def _gather_request(inp, b, Hkv, D):
    """Dense [1, Hkv, kv_len, D] K/V of request b, gathered page by page."""
    ps = inp.page_size
    p0, p1 = int(inp.kv_indptr[b]), int(inp.kv_indptr[b + 1])
    n = 0 if p1 == p0 else (p1 - p0 - 1) * ps + int(inp.kv_last_page_len[b])
    pages = inp.kv_indices[p0:p1].long()
    kd = inp.k_cache[pages].reshape(-1, Hkv, D)[:n].permute(1, 0, 2).unsqueeze(0).contiguous()
    vd = inp.v_cache[pages].reshape(-1, Hkv, D)[:n].permute(1, 0, 2).unsqueeze(0).contiguous()
    return kd, vd


@pytest.mark.parametrize("page_size,causal,dtype", [(1, True, "f32"), (4, True, "bf16"), (8, False, "f32"),
                                                    (16, True, "f16")])
def test_paged_prefill_matches_torch_reference_per_request(page_size, causal, dtype):
    # Every request against torch fp64 over its own gathered K/V; the lengths
    # include empty requests, requests with no keys, q_len > kv_len (leading
    # rows see nothing) and partly filled last pages.
    q_lens = [3, 0, 5, 7, 1, 4]
    kv_lens = [9, 4, 0, 3, 17, 4]
    inp = make_paged_prefill(6, 8, 2, 16, dtype, seed=40 + page_size, page_size=page_size,
                             q_lens=q_lens, kv_lens=kv_lens)
    o, l = oracle.attn_prefill_paged(inp.q, inp.k_cache, inp.v_cache, inp.qo_indptr, inp.kv_indptr,
                                     inp.kv_indices, 0.3, causal, inp.kv_last_page_len)
    for b in range(6):
        t0, t1 = int(inp.qo_indptr[b]), int(inp.qo_indptr[b + 1])
        if t1 == t0:
            continue
        kd, vd = _gather_request(inp, b, 2, 16)
        qd = inp.q[t0:t1].permute(1, 0, 2).unsqueeze(0).contiguous()   # [1, Hq, q_len, D]
        o_ref, l_ref = torch_reference(qd, kd, vd, 0.3, causal)
        np.testing.assert_allclose(o[t0:t1], o_ref[0].transpose(1, 0, 2), atol=TOL, rtol=0)
        lr = l_ref[0].T
        np.testing.assert_array_equal(np.isneginf(l[t0:t1]), np.isneginf(lr))
        fin = np.isfinite(lr)
        np.testing.assert_allclose(l[t0:t1][fin], lr[fin], atol=TOL, rtol=0)


def test_paged_prefill_equals_dense_forward():
    # One request with a full page table is the dense forward over the same K/V.
    inp = make_paged_prefill(1, 4, 2, 32, "bf16", seed=47, page_size=8, q_lens=[13], kv_lens=[29])
    kd, vd = _gather_request(inp, 0, 2, 32)
    qd = inp.q.permute(1, 0, 2).unsqueeze(0).contiguous()
    o1, l1 = oracle.attn_prefill_paged(inp.q, inp.k_cache, inp.v_cache, inp.qo_indptr, inp.kv_indptr,
                                       inp.kv_indices, 0.2, True, inp.kv_last_page_len)
    o2, l2 = oracle.attn_fwd(qd, kd, vd, 0.2, True)
    assert np.array_equal(o1, o2[0].transpose(1, 0, 2)) and np.array_equal(l1, l2[0].T)


# ---- decode over an 8-bit E4M3 cache ---------------------------------------------

def test_widen_every_e4m3_pattern():
    b = torch.arange(256, dtype=torch.uint8)
    got = oracle.widen(b, fp8=True)
    ref = b.view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(ref)], ref[~np.isnan(ref)])


def _dequant(x8, ss):
    """x8 * scale + shift in fp64, with torch's own E4M3 and fp16 decoding."""
    ss = ss.to(torch.int32)
    sc = (ss & 0xFFFF).to(torch.int16).view(torch.float16).double()
    sh = ((ss >> 16) & 0xFFFF).to(torch.int16).view(torch.float16).double()
    return x8.view(torch.float8_e4m3fn).double() * sc[..., None] + sh[..., None]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_fp8_matches_torch_on_dequantized_cache(dtype):
    inp = make_decode_fp8(3, 8, 2, 16, dtype, seed=60, len_lo=1, len_hi=40, page_size=8)
    o, l = oracle.attn_decode_fp8(inp.q, inp.k8, inp.v8, inp.k_ss, inp.v_ss, inp.seq_lens, 0.25,
                                  block_table=inp.block_table)
    kd_all, vd_all = _dequant(inp.k8, inp.k_ss), _dequant(inp.v8, inp.v_ss)
    for b in range(3):
        n = int(inp.seq_lens[b])
        pages = inp.block_table[b, :(n + 7) // 8].long()
        kd = kd_all[pages].reshape(-1, 2, 16)[:n].permute(1, 0, 2).unsqueeze(0).contiguous()
        vd = vd_all[pages].reshape(-1, 2, 16)[:n].permute(1, 0, 2).unsqueeze(0).contiguous()
        o_ref, l_ref = torch_reference(inp.q[b].view(1, 8, 1, 16), kd, vd, 0.25, True)
        np.testing.assert_allclose(o[b], o_ref[0, :, 0], atol=TOL, rtol=0)
        np.testing.assert_allclose(l[b], l_ref[0, :, 0], atol=TOL, rtol=0)


def test_decode_fp8_unit_scale_is_plain_decode():
    # scale 1, shift 0: the E4M3 values themselves, which bf16 holds exactly
    inp = make_decode_fp8(2, 4, 2, 32, "bf16", seed=61, len_lo=5, len_hi=50, page_size=16)
    one = torch.full_like(inp.k_ss, 0x3C00)  # fp16 1.0 in bits 0-15, +0.0 in bits 16-31
    o1, l1 = oracle.attn_decode_fp8(inp.q, inp.k8, inp.v8, one, one, inp.seq_lens, 0.2,
                                    block_table=inp.block_table)
    kb = inp.k8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    vb = inp.v8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    o2, l2 = oracle.attn_decode(inp.q, kb, vb, inp.seq_lens, 0.2, block_table=inp.block_table)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---- additive bias (splitk_kernels.py, `_fwd_kernel_splitK` HAS_ADDITIVE_BIAS) ----

def torch_reference_bias(q, k, v, bias, scale, causal):
    """softmax(scale * Q K^T + bias + mask) V in torch fp64; a row whose
    visible scores are all -inf gives (0, -inf)."""
    q, k, v = (t.to(torch.float64) for t in (q, k, v))
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    k = k.repeat_interleave(G, dim=1)
    v = v.repeat_interleave(G, dim=1)
    s = scale * torch.matmul(q, k.transpose(-1, -2).contiguous()) + bias.to(torch.float64)
    if causal:
        i = torch.arange(Lq).view(-1, 1)
        j = torch.arange(Lk).view(1, -1)
        s = s.masked_fill(~(j <= i + (Lk - Lq)), float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    empty = torch.isneginf(lse)
    p = torch.softmax(s, dim=-1)
    p = torch.where(empty[..., None], torch.zeros_like(p), p)
    return torch.matmul(p, v).numpy(), lse.numpy()


BIAS_SHAPES = [
    # B, Hq, Hkv, q_len, kv_len, D, causal, bias shape (broadcast dims = 1)
    (1, 2, 1, 5, 5, 8, True, "full"),
    (2, 4, 2, 7, 9, 16, False, "full"),
    (1, 4, 2, 6, 11, 8, True, "per_head"),      # [1, Hq, q_len, kv_len]: shared by the batch
    (2, 8, 2, 9, 4, 8, True, "per_batch"),      # [B, 1, q_len, kv_len]: shared by the heads
    (1, 6, 3, 3, 13, 32, False, "keys_only"),   # [1, 1, 1, kv_len]: one row for every query
]


def _bias_of(kind, B, Hq, Lq, Lk, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    shape = {"full": (B, Hq, Lq, Lk), "per_head": (1, Hq, Lq, Lk), "per_batch": (B, 1, Lq, Lk),
             "keys_only": (1, 1, 1, Lk)}[kind]
    return (2.0 * torch.randn(shape, generator=g)).to(dtype)


@pytest.mark.parametrize("shape", BIAS_SHAPES)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_bias_matches_torch(shape, dtype):
    B, Hq, Hkv, Lq, Lk, D, causal, kind = shape
    q, k, v = make_prefill(B, Hq, Hkv, Lq, Lk, D, dtype, seed=Lq * Lk + D)
    bias = _bias_of(kind, B, Hq, Lq, Lk, q.dtype, seed=D)
    scale = fp32_scale(D)
    o, lse = oracle.attn_fwd_bias(q, k, v, bias, scale, causal)
    o_ref, lse_ref = torch_reference_bias(q, k, v, bias.expand(B, Hq, Lq, Lk), scale, causal)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=TOL)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=0, atol=TOL)


def test_zero_bias_is_no_bias_bitwise():
    q, k, v = make_prefill(2, 4, 2, 9, 13, 16, "bf16", seed=3)
    for causal in (True, False):
        o1, l1 = oracle.attn_fwd(q, k, v, 0.25, causal)
        o2, l2 = oracle.attn_fwd_bias(q, k, v, torch.zeros(1, 1, 1, 1), 0.25, causal)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_minus_inf_bias_on_the_causal_pattern_is_causal():
    # a bias of -inf exactly where the bottom-right rule hides a key, 0 elsewhere,
    # without the causal flag: the causal result (also for q_len > kv_len rows)
    for Lq, Lk in ((7, 7), (5, 12), (9, 4)):
        q, k, v = make_prefill(1, 4, 2, Lq, Lk, 8, "f32", seed=Lq + Lk)
        i = torch.arange(Lq).view(-1, 1)
        j = torch.arange(Lk).view(1, -1)
        bias = torch.where(j <= i + (Lk - Lq), 0.0, float("-inf")).view(1, 1, Lq, Lk)
        o1, l1 = oracle.attn_fwd(q, k, v, 0.3, True)
        o2, l2 = oracle.attn_fwd_bias(q, k, v, bias, 0.3, False)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_bias_as_log_weights_with_zero_keys():
    # K = 0 makes every score 0, so bias_ij = log w_ij gives P_ij = w_ij / sum_j w_ij:
    # O_i = sum_j w_ij v_j / sum_j w_ij and L_i = log sum_j w_ij (closed form; a
    # transposed or mis-strided bias index would pick other weights)
    B, Hq, Hkv, Lq, Lk, D = 2, 4, 2, 5, 9, 8
    _, _, v = make_prefill(B, Hq, Hkv, Lq, Lk, D, "f32", seed=11)
    q = torch.randn(B, Hq, Lq, D)
    k = torch.zeros(B, Hkv, Lk, D)
    g = torch.Generator().manual_seed(12)
    w = torch.rand(B, Hq, Lq, Lk, generator=g, dtype=torch.float64) + 0.1
    o, lse = oracle.attn_fwd_bias(q, k, v, torch.log(w), 0.7, False)
    vv = v.double().repeat_interleave(Hq // Hkv, dim=1)
    o_ref = torch.matmul(w, vv) / w.sum(-1, keepdim=True)
    np.testing.assert_allclose(o, o_ref.numpy(), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, torch.log(w.sum(-1)).numpy(), rtol=0, atol=1e-13)


def test_row_constant_bias_shifts_lse_only():
    q, k, v = make_prefill(1, 4, 2, 6, 10, 16, "f32", seed=21)
    c = torch.tensor([0.5, -3.0, 7.25, 0.0, 1.0, -0.125], dtype=torch.float64).view(1, 1, 6, 1)
    o1, l1 = oracle.attn_fwd(q, k, v, 0.2, True)
    o2, l2 = oracle.attn_fwd_bias(q, k, v, c, 0.2, True)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + c.view(1, 1, 6).numpy(), rtol=0, atol=1e-13)


def test_bias_masking_every_key_gives_empty_row():
    q, k, v = make_prefill(1, 2, 1, 3, 5, 8, "f32", seed=2)
    bias = torch.zeros(1, 2, 3, 5)
    bias[0, 1, 2, :] = float("-inf")
    o, lse = oracle.attn_fwd_bias(q, k, v, bias, 0.3, False)
    assert np.all(o[0, 1, 2] == 0) and lse[0, 1, 2] == -np.inf
    assert np.isfinite(lse[0, 0]).all() and np.isfinite(lse[0, 1, :2]).all()


@pytest.mark.parametrize("q_len", [1, 3])
def test_decode_bias_matches_torch_on_gathered_keys(q_len):
    inp = make_decode(3, 8, 2, 16, "bf16", seed=31 + q_len, len_lo=1, len_hi=40, page_size=8, q_len=q_len)
    scale = fp32_scale(16)
    L = int(inp.seq_lens.max())
    g = torch.Generator().manual_seed(5)
    bias = torch.randn(3, 8, q_len, L, generator=g).to(torch.bfloat16)
    q4 = inp.q if inp.q.dim() == 4 else inp.q.unsqueeze(2)
    o, lse = oracle.attn_decode_bias(q4, inp.k_cache, inp.v_cache, inp.seq_lens, bias, scale,
                                     block_table=inp.block_table, max_kv_len=inp.max_kv_len)
    for b in range(3):
        n = int(inp.seq_lens[b])
        pages = inp.block_table[b, :(n + 7) // 8].long()
        kd = inp.k_cache[pages].reshape(-1, 2, 16)[:n].permute(1, 0, 2).unsqueeze(0)
        vd = inp.v_cache[pages].reshape(-1, 2, 16)[:n].permute(1, 0, 2).unsqueeze(0)
        # the q_len queries are the last positions: a causal forward with kv_len = n
        o_ref, l_ref = torch_reference_bias(q4[b:b + 1], kd, vd, bias[b:b + 1, :, :, :n], scale, True)
        np.testing.assert_allclose(o[b], o_ref[0], rtol=0, atol=TOL)
        fin = np.isfinite(l_ref[0])
        assert np.array_equal(fin, np.isfinite(lse[b]))
        np.testing.assert_allclose(lse[b][fin], l_ref[0][fin], rtol=0, atol=TOL)


def test_decode_bias_equals_prefill_bias_for_one_query():
    q, k, v = make_prefill(2, 4, 2, 1, 23, 8, "f32", seed=8)
    bias = torch.randn(2, 4, 1, 23, dtype=torch.float64)
    o1, l1 = oracle.attn_fwd_bias(q, k, v, bias, 0.4, False)
    lens = torch.tensor([23, 23], dtype=torch.int32)
    o2, l2 = oracle.attn_decode_bias(q, k, v, lens, bias, 0.4)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-15)


# ---- merge of partial results and its backward (splitk_kernels.py,
# `_splitK_reduce` and `_splitK_reduce_varargs_backward`) ----------------------

def _partials(rows, S, D, seed, empty=()):
    g = np.random.default_rng(seed)
    op = g.standard_normal((rows, S, D))
    lp = 3.0 * g.standard_normal((rows, S))
    for r, s in empty:
        op[r, s] = 0.0
        lp[r, s] = -np.inf
    return op, lp


def test_merge_equals_unsplit_attention():
    # split the keys of plain attention rows into chunks, merge: the unsplit row
    q, k, v = make_prefill(1, 2, 1, 3, 20, 8, "f32", seed=4)
    edges = [0, 5, 6, 13, 20]
    parts = [oracle.attn_fwd(q, k[:, :, a:b], v[:, :, a:b], 0.3, False) for a, b in zip(edges, edges[1:])]
    op = np.stack([p[0] for p in parts], axis=-2)
    lp = np.stack([p[1] for p in parts], axis=-1)
    o, lse = oracle.splitk_merge(op, lp)
    o_ref, l_ref = oracle.attn_fwd(q, k, v, 0.3, False)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, l_ref, rtol=0, atol=1e-14)


def _objective(op, lp, d_o, d_lse):
    o, lse = oracle.splitk_merge(op, lp)
    return float((o * d_o).sum() + (lse * d_lse).sum())


def test_merge_backward_matches_finite_differences():
    rows, S, D = 3, 4, 5
    op, lp = _partials(rows, S, D, seed=1, empty=[(1, 2)])
    g = np.random.default_rng(2)
    d_o, d_lse = g.standard_normal((rows, D)), g.standard_normal(rows)
    o, lse = oracle.splitk_merge(op, lp)
    dop, dlp = oracle.splitk_merge_backward(op, lp, o, lse, d_o, d_lse)
    h = 1e-6
    for r in range(rows):
        for s in range(S):
            if np.isneginf(lp[r, s]):
                continue
            for d in range(D):
                a, b = op.copy(), op.copy()
                a[r, s, d] += h
                b[r, s, d] -= h
                fd = (_objective(a, lp, d_o, d_lse) - _objective(b, lp, d_o, d_lse)) / (2 * h)
                assert abs(fd - dop[r, s, d]) <= 1e-7 * (1 + abs(fd))
            a, b = lp.copy(), lp.copy()
            a[r, s] += h
            b[r, s] -= h
            fd = (_objective(op, a, d_o, d_lse) - _objective(op, b, d_o, d_lse)) / (2 * h)
            assert abs(fd - dlp[r, s]) <= 1e-7 * (1 + abs(fd))
    # an empty chunk has weight 0 and gets no gradient
    assert np.all(dop[1, 2] == 0) and dlp[1, 2] == 0


def test_merge_backward_sums_and_single_split():
    rows, S, D = 6, 5, 7
    op, lp = _partials(rows, S, D, seed=3, empty=[(0, 0), (0, 4), (2, 1)])
    g = np.random.default_rng(4)
    d_o, d_lse = g.standard_normal((rows, D)), g.standard_normal(rows)
    o, lse = oracle.splitk_merge(op, lp)
    dop, dlp = oracle.splitk_merge_backward(op, lp, o, lse, d_o, d_lse)
    # the weights sum to 1 and sum_s w_s (O_s - O) = 0: the gradients of the
    # partials add up to the incoming ones
    np.testing.assert_allclose(dop.sum(axis=1), d_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dlp.sum(axis=1), d_lse, rtol=0, atol=1e-13)
    # one split: the merge is the identity
    o1, l1 = oracle.splitk_merge(op[:, :1], lp[:, :1])
    d1, dl1 = oracle.splitk_merge_backward(op[:, :1], lp[:, :1], o1, l1, d_o, d_lse)
    fin = np.isfinite(lp[:, 0])
    np.testing.assert_allclose(d1[fin, 0], d_o[fin], rtol=0, atol=1e-15)
    np.testing.assert_allclose(dl1[fin, 0], d_lse[fin], rtol=0, atol=1e-15)


def test_merge_backward_equal_lse_gives_equal_weights():
    # S partials with one LSE: w_s = 1/S, dO_s = dO/S, dL_s = (dL + <O_s - O, dO>)/S
    S, D = 4, 3
    op = np.arange(S * D, dtype=np.float64).reshape(1, S, D) / 7.0
    lp = np.full((1, S), 0.75)
    d_o, d_lse = np.array([[1.0, -2.0, 0.5]]), np.array([0.25])
    o, lse = oracle.splitk_merge(op, lp)
    np.testing.assert_allclose(o[0], op[0].mean(axis=0), rtol=0, atol=1e-15)
    assert abs(lse[0] - (0.75 + math.log(S))) <= 1e-15
    dop, dlp = oracle.splitk_merge_backward(op, lp, o, lse, d_o, d_lse)
    np.testing.assert_allclose(dop[0], np.tile(d_o / S, (S, 1)), rtol=0, atol=1e-15)
    want = (d_lse[0] + ((op[0] - o[0]) * d_o[0]).sum(axis=1)) / S
    np.testing.assert_allclose(dlp[0], want, rtol=0, atol=1e-14)


def test_merge_backward_all_empty_row_is_zero():
    op, lp = _partials(2, 3, 4, seed=9, empty=[(0, 0), (0, 1), (0, 2)])
    o, lse = oracle.splitk_merge(op, lp)
    assert lse[0] == -np.inf and np.all(o[0] == 0)
    dop, dlp = oracle.splitk_merge_backward(op, lp, o, lse, np.ones((2, 4)), np.ones(2))
    assert np.all(dop[0] == 0) and np.all(dlp[0] == 0)
    assert np.isfinite(dop[1]).all() and np.isfinite(dlp[1]).all()
