"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented status codes
before launching anything.  No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import gqa_attention_forward_attn_amd as gqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")
TEST_HEADER = os.path.join(ROOT, "include", "gqa_attn_test.h")
CEILING_HEADER = os.path.join(ROOT, "include", "gqa_ceilings.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, 1, 2, 3, 4
BF16, F16, F32 = gqa.GQA_BF16, gqa.GQA_F16, gqa.GQA_F32
# Fake, 256-byte aligned device addresses: validation rejects every call
# below before any pointer is used.
P = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(8)]


def declared_functions(path=HEADER):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof"})


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gqa.LIB_PATH):
        pytest.fail("libgqa_attn.so is not built (run __graft_entry__.build())")
    return gqa.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(gqa.EXPORTS)
    for n in names:
        assert hasattr(L, n), f"{n} declared in gqa_attn.h but not exported"
    test_names = declared_functions(TEST_HEADER)
    assert set(test_names) == set(gqa.TEST_EXPORTS)
    for n in test_names:
        assert hasattr(L, n), f"{n} declared in gqa_attn_test.h but not exported"
    ceiling_names = declared_functions(CEILING_HEADER)
    assert set(ceiling_names) == set(gqa.CEILING_EXPORTS)
    for n in ceiling_names:
        assert hasattr(L, n), f"{n} declared in gqa_ceilings.h but not exported"


def test_noalloc_decode_rejects_requests_beyond_its_scratch(L):
    # B * Hq * n_splits * (D + 1) * 4 bytes above the fixed 32 MiB: refused
    # before any HIP call (so this runs without a GPU)
    p = [P[i] for i in range(7)]
    assert L.attn_decode_splitk_noalloc(*p, 4, 256, 1024, 32, 8, 128, 1024, 0.088, 16, BF16, None) == WORKSPACE
    assert L.attn_decode_splitk_noalloc(*p, 4, 256, 128, 32, 8, 128, 1024, 0.088, 16, BF16, None) == WORKSPACE  # 33.8 MB


def test_bias_and_merge_backward_validation(L):
    args = (P[0], P[1], P[2], P[5])
    # attn_fwd_bias: strides >= 0, a bias pointer, 16-bit dtypes only
    assert L.attn_fwd_bias(*args, 0, 0, 8, P[3], P[4], 1, 4, 2, 8, 8, 64, 0.125, 1, F32, None) == UNSUPPORTED
    assert L.attn_fwd_bias(*args, -1, 0, 8, P[3], P[4], 1, 4, 2, 8, 8, 64, 0.125, 1, BF16, None) == INVALID
    assert L.attn_fwd_bias(P[0], P[1], P[2], None, 0, 0, 8, P[3], P[4], 1, 4, 2, 8, 8, 64, 0.125, 1, BF16,
                           None) == INVALID
    assert L.attn_fwd_bias(P[0], P[1], P[2], ctypes.c_void_p(0x10001), 0, 0, 8, P[3], P[4], 1, 4, 2, 8, 8, 64,
                           0.125, 1, BF16, None) == INVALID          # bias not 2-byte aligned
    assert L.attn_fwd_bias(*args, 0, 0, 8, P[3], P[4], 0, 4, 2, 8, 8, 64, 0.125, 1, BF16, None) == OK
    # attn_decode_splitk_bias: even strides, 4-byte aligned bias
    d = (P[0], P[1], P[2], P[5])
    rest = (P[3], P[4], P[6], P[7], 4, 16, 2, 8, 2, 1, 64, 64, 0.125, 4, P[7], 1 << 20, BF16, None)
    assert L.attn_decode_splitk_bias(*d, 0, 0, 7, *rest) == INVALID
    assert L.attn_decode_splitk_bias(*d, 0, -2, 8, *rest) == INVALID
    assert L.attn_decode_splitk_bias(P[0], P[1], P[2], ctypes.c_void_p(0x10002), 0, 0, 8, *rest) == INVALID
    # merge backward: sizes
    m = [P[i] for i in range(8)]
    assert L.attn_splitk_merge_backward(*m, 0, 16, 128, None) == OK
    assert L.attn_splitk_merge_backward(*m, 10, 0, 128, None) == INVALID
    assert L.attn_splitk_merge_backward(*m, 10, 16, 0, None) == INVALID
    assert L.attn_splitk_merge_backward(*m, 10, 16, 513, None) == INVALID
    assert L.attn_splitk_merge_backward(*m, -1, 16, 128, None) == INVALID
    m[3] = None
    assert L.attn_splitk_merge_backward(*m, 10, 16, 128, None) == INVALID


def test_ceiling_validation(L):
    assert L.gqa_ceiling_mfma_flops(256, 100) == 256 * 8 * 100 * 16 * 32768
    assert L.gqa_ceiling_mfma_flops(0, 100) == 0
    assert L.gqa_ceiling_mfma(0, 10, P[0], None) == 1
    assert L.gqa_ceiling_mfma(4, 10, None, None) == 1
    assert L.gqa_ceiling_stream_read(P[0], 24, 4, P[1], None) == 1    # not a multiple of 16
    assert L.gqa_ceiling_stream_read(ctypes.c_void_p(0x10008), 64, 4, P[1], None) == 1   # misaligned


def test_kernel_choice_validation(L):
    # the test entry points reject an unknown kernel code before anything else
    args = (P[0], P[1], P[2], P[3], P[4], 1, 4, 2, 8, 8, 64, 0.125, 1, BF16)
    assert L.attn_fwd_with_kernel(*args, 3, None) == INVALID
    assert L.attn_fwd_with_kernel(*args, -1, None) == INVALID
    assert L.attn_fwd_with_kernel(P[0], P[1], P[2], P[3], P[4], 0, 4, 2, 8, 8, 64, 0.125, 1, BF16, 2, None) == OK


def test_status_strings(L):
    for code in range(5):
        s = L.attn_status_str(code).decode()
        assert s.startswith(gqa.STATUS[code])
    assert L.attn_status_str(99).decode().startswith("unknown")


def test_workspace_bytes(L):
    assert L.attn_decode_workspace_bytes(16, 32, 128, 16) == 16 * 32 * 16 * 129 * 4
    assert L.attn_decode_workspace_bytes(0, 32, 128, 16) == 0
    assert L.attn_decode_workspace_bytes(1, 1, 64, 0) == 0


def fwd(L, B=1, Hq=4, Hkv=2, q_len=8, kv_len=8, D=64, scale=0.125, causal=1, dtype=BF16,
        q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4]):
    return L.attn_fwd(q, k, v, o, lse, B, Hq, Hkv, q_len, kv_len, D, scale, causal, dtype, None)


def test_fwd_validation(L):
    assert fwd(L, Hq=6, Hkv=4) == INVALID          # Hq % Hkv
    assert fwd(L, Hkv=0) == INVALID
    assert fwd(L, B=-1) == INVALID
    assert fwd(L, q_len=-3) == INVALID
    assert fwd(L, kv_len=-1) == INVALID
    assert fwd(L, scale=float("nan")) == INVALID
    assert fwd(L, scale=0.0) == INVALID
    assert fwd(L, dtype=7) == INVALID
    assert fwd(L, D=96) == UNSUPPORTED
    assert fwd(L, D=256) == UNSUPPORTED
    assert fwd(L, q=None) == INVALID
    assert fwd(L, lse=None) == INVALID
    assert fwd(L, k=None) == INVALID
    assert fwd(L, q=ctypes.c_void_p(0x10008)) == INVALID   # misaligned
    # nothing to do: returns OK without launching
    assert fwd(L, B=0) == OK
    assert fwd(L, q_len=0) == OK


def fwd_split(L, kv_splits=2, ws=P[7], ws_bytes=None, B=1, Hq=4, Hkv=2, q_len=8, kv_len=8, D=64, dtype=BF16,
              q=P[0]):
    if ws_bytes is None:
        ws_bytes = L.attn_fwd_split_workspace_bytes(B, Hq, q_len, D, kv_splits)
    return L.attn_fwd_split(q, P[1], P[2], P[3], P[4], B, Hq, Hkv, q_len, kv_len, D, 0.125, 1, kv_splits,
                            ws, ws_bytes, dtype, None)


def test_fwd_split_workspace_and_validation(L):
    # fp32 partial outputs [B, Hq, q_len, kv_splits, D] then partial LSEs
    assert L.attn_fwd_split_workspace_bytes(1, 32, 1024, 128, 2) == 32 * 1024 * 2 * 129 * 4
    assert L.attn_fwd_split_workspace_bytes(1, 32, 1024, 128, 1) == 0
    assert L.attn_fwd_split_workspace_bytes(0, 32, 1024, 128, 2) == 0
    assert fwd_split(L, kv_splits=0) == INVALID
    assert fwd_split(L, kv_splits=65) == INVALID
    assert fwd_split(L, Hq=6, Hkv=4) == INVALID
    assert fwd_split(L, D=96) == UNSUPPORTED
    assert fwd_split(L, dtype=F32) == UNSUPPORTED
    assert fwd_split(L, ws=None) == WORKSPACE
    assert fwd_split(L, ws_bytes=16) == WORKSPACE
    assert fwd_split(L, ws=ctypes.c_void_p(0x20008)) == WORKSPACE   # misaligned
    assert fwd_split(L, q=None) == INVALID
    assert fwd_split(L, B=0) == OK
    # kv_splits = 1 is attn_fwd itself (no workspace needed)
    assert fwd_split(L, kv_splits=1, ws=None, ws_bytes=0, B=0) == OK
    assert fwd_split(L, kv_splits=1, ws=None, ws_bytes=0, Hq=6, Hkv=4) == INVALID


def test_fwd_kv_splits_recommendation(L):
    # never for fp32, short key ranges or bad geometry; without a device (host
    # only) the CU count is unknown and the answer is 1
    assert L.attn_fwd_kv_splits(1, 32, 4, 1024, 4096, 128, 1, F32) == 1
    assert L.attn_fwd_kv_splits(1, 32, 4, 1024, 1024, 128, 1, BF16) == 1
    assert L.attn_fwd_kv_splits(1, 6, 4, 1024, 4096, 128, 1, BF16) == 1
    assert L.attn_fwd_kv_splits(1, 32, 4, 1024, 4096, 96, 1, BF16) == 1
    assert L.attn_fwd_kv_splits(1, 32, 4, 1024, 4096, 128, 1, BF16) >= 1


def dec(L, B=2, Hq=8, Hkv=2, D=128, max_kv_len=512, n_splits=4, page_size=256, max_pages=2,
        bt=P[6], ws=P[7], ws_bytes=None, dtype=BF16, scale=0.1, q=P[0], seq=P[5]):
    if ws_bytes is None:
        ws_bytes = L.attn_decode_workspace_bytes(B, Hq, D, n_splits)
    return L.attn_decode_splitk(q, P[1], P[2], P[3], P[4], seq, bt, max_pages, page_size,
                                B, Hq, Hkv, D, max_kv_len, scale, n_splits, ws, ws_bytes,
                                dtype, None)


def test_decode_validation(L):
    assert dec(L, Hq=6, Hkv=4) == INVALID
    assert dec(L, n_splits=0) == INVALID
    assert dec(L, n_splits=257) == INVALID
    assert dec(L, page_size=96) == INVALID             # not a power of two
    assert dec(L, page_size=0) == INVALID
    assert dec(L, max_pages=1) == INVALID              # 1 * 256 < max_kv_len
    assert dec(L, scale=-1.0) == INVALID
    assert dec(L, max_kv_len=-1) == INVALID
    assert dec(L, D=80) == UNSUPPORTED
    assert dec(L, dtype=F32) == UNSUPPORTED
    assert dec(L, q=None) == INVALID
    assert dec(L, seq=None) == INVALID
    assert dec(L, ws=None) == WORKSPACE
    assert dec(L, ws_bytes=100) == WORKSPACE
    assert dec(L, B=0) == OK


def test_workspace_bytes_multi(L):
    assert L.attn_decode_workspace_bytes_multi(16, 32, 4, 128, 16) == 16 * 32 * 4 * 16 * 129 * 4
    assert L.attn_decode_workspace_bytes_multi(16, 32, 1, 128, 16) == L.attn_decode_workspace_bytes(16, 32, 128, 16)
    assert L.attn_decode_workspace_bytes_multi(2, 8, 0, 128, 4) == 0


def dec_multi(L, B=2, Hq=8, Hkv=2, q_len=4, D=128, max_kv_len=512, n_splits=4, page_size=256, max_pages=2,
              bt=P[6], ws=P[7], ws_bytes=None, dtype=BF16, scale=0.1, q=P[0], seq=P[5]):
    if ws_bytes is None:
        ws_bytes = L.attn_decode_workspace_bytes_multi(B, Hq, max(q_len, 1), D, n_splits)
    return L.attn_decode_splitk_multi(q, P[1], P[2], P[3], P[4], seq, bt, max_pages, page_size,
                                      B, Hq, Hkv, q_len, D, max_kv_len, scale, n_splits, ws, ws_bytes,
                                      dtype, None)


def test_decode_multi_validation(L):
    assert dec_multi(L, q_len=0) == INVALID
    assert dec_multi(L, q_len=257) == INVALID
    assert dec_multi(L, Hq=6, Hkv=4) == INVALID
    assert dec_multi(L, n_splits=0) == INVALID
    assert dec_multi(L, page_size=96) == INVALID
    assert dec_multi(L, D=80) == UNSUPPORTED
    assert dec_multi(L, dtype=F32) == UNSUPPORTED
    assert dec_multi(L, q=None) == INVALID
    # the workspace of one query per sequence is too small for four
    assert dec_multi(L, ws_bytes=L.attn_decode_workspace_bytes(2, 8, 128, 4)) == WORKSPACE
    assert dec_multi(L, ws=None) == WORKSPACE
    assert dec_multi(L, B=0) == OK


def pre_paged(L, B=2, Hq=8, Hkv=2, D=128, page_size=16, max_q_len=64, scale=0.1, causal=1, dtype=BF16,
              q=P[0], qo=P[5], kvp=P[6], idx=P[7], last=None):
    return L.attn_prefill_paged(q, P[1], P[2], P[3], P[4], qo, kvp, idx, last, B, Hq, Hkv, D, page_size,
                                max_q_len, scale, causal, dtype, None)


def test_prefill_paged_validation(L):
    assert pre_paged(L, Hq=6, Hkv=4) == INVALID
    assert pre_paged(L, page_size=24) == INVALID        # not a power of two
    assert pre_paged(L, page_size=0) == INVALID
    assert pre_paged(L, max_q_len=-1) == INVALID
    assert pre_paged(L, scale=float("inf")) == INVALID
    assert pre_paged(L, dtype=9) == INVALID
    assert pre_paged(L, D=96) == UNSUPPORTED
    assert pre_paged(L, dtype=F32) == UNSUPPORTED
    assert pre_paged(L, q=None) == INVALID
    assert pre_paged(L, idx=None) == INVALID
    assert pre_paged(L, qo=None) == INVALID
    assert pre_paged(L, q=ctypes.c_void_p(0x10004)) == INVALID   # misaligned
    assert pre_paged(L, B=0) == OK
    assert pre_paged(L, max_q_len=0) == OK


def dec_fp8(L, B=2, Hq=8, Hkv=2, D=128, max_kv_len=512, n_splits=4, page_size=256, max_pages=2,
            bt=P[6], ws=P[7], ws_bytes=None, dtype=BF16, scale=0.1, q=P[0], seq=P[5], kss=P[1], vss=P[2]):
    if ws_bytes is None:
        ws_bytes = L.attn_decode_workspace_bytes(B, Hq, D, n_splits)
    return L.attn_decode_splitk_fp8(q, P[1], P[2], kss, vss, P[3], P[4], seq, bt, max_pages, page_size,
                                    B, Hq, Hkv, D, max_kv_len, scale, n_splits, ws, ws_bytes, dtype, None)


def test_decode_fp8_validation(L):
    assert dec_fp8(L, Hq=6, Hkv=4) == INVALID
    assert dec_fp8(L, n_splits=0) == INVALID
    assert dec_fp8(L, page_size=96) == INVALID
    assert dec_fp8(L, page_size=8, max_pages=64) == UNSUPPORTED   # a page must hold a 16-token slice
    assert dec_fp8(L, D=80) == UNSUPPORTED
    assert dec_fp8(L, dtype=F32) == UNSUPPORTED
    assert dec_fp8(L, kss=None) == INVALID
    assert dec_fp8(L, vss=ctypes.c_void_p(0x20002)) == INVALID  # scale-shift words need 4-byte alignment
    assert dec_fp8(L, ws=None) == WORKSPACE
    assert dec_fp8(L, B=0) == OK


def test_python_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gqa.attn_fwd(q, q[:, :1].contiguous(), q[:, :1].contiguous())
