"""Python binding of libgqa_attn.so (the C ABI in include/gqa_attn.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback path: if the library is not built, or a call returns an
error status, these functions raise.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgqa_attn.so")

GQA_F32, GQA_F16, GQA_BF16 = 0, 1, 2
STATUS = {0: "GQA_OK", 1: "GQA_ERR_INVALID_ARG", 2: "GQA_ERR_UNSUPPORTED",
          3: "GQA_ERR_WORKSPACE", 4: "GQA_ERR_HIP"}
_TORCH_DT = {torch.float32: GQA_F32, torch.float16: GQA_F16, torch.bfloat16: GQA_BF16}

# Every symbol include/gqa_attn.h declares.
EXPORTS = ("attn_fwd", "attn_fwd_bias", "attn_fwd_split", "attn_fwd_split_workspace_bytes", "attn_fwd_kv_splits",
           "attn_prefill_paged", "attn_decode_workspace_bytes", "attn_decode_splitk",
           "attn_decode_splitk_fp8",
           "attn_decode_workspace_bytes_multi", "attn_decode_splitk_multi", "attn_decode_splitk_noalloc",
           "attn_decode_splitk_bias", "attn_splitk_merge_backward", "attn_status_str")
# Every symbol include/gqa_attn_test.h declares (kernel selection for tests).
TEST_EXPORTS = ("attn_fwd_with_kernel", "attn_prefill_paged_with_kernel")
# Every symbol include/gqa_ceilings.h declares (measurement kernels).
CEILING_EXPORTS = ("gqa_ceiling_mfma_flops", "gqa_ceiling_mfma", "gqa_ceiling_stream_read")
# bf16 / fp16 prefill kernel names accepted by the `kernel` argument
PREFILL_KERNELS = {None: 0, "auto": 0, "pingpong": 1, "fourwave": 2}

_lib = None


class GqaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded C library with argument types declared (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                           "python -m gqa_attention_forward_attn_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, vp]
    L.attn_fwd.restype = i32
    i64 = ctypes.c_longlong
    L.attn_fwd_bias.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, vp]
    L.attn_fwd_bias.restype = i32
    L.attn_fwd_with_kernel.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, i32, vp]
    L.attn_fwd_with_kernel.restype = i32
    L.attn_fwd_split.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, vp, sz, i32, vp]
    L.attn_fwd_split.restype = i32
    L.attn_fwd_split_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    L.attn_fwd_split_workspace_bytes.restype = sz
    L.attn_fwd_kv_splits.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    L.attn_fwd_kv_splits.restype = i32
    L.attn_prefill_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                     f32, i32, i32, vp]
    L.attn_prefill_paged.restype = i32
    L.attn_prefill_paged_with_kernel.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                 i32, f32, i32, i32, i32, vp]
    L.attn_prefill_paged_with_kernel.restype = i32
    L.attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_decode_splitk.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                     f32, i32, vp, sz, i32, vp]
    L.attn_decode_splitk.restype = i32
    L.attn_decode_splitk_bias.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                          i32, i32, i32, f32, i32, vp, sz, i32, vp]
    L.attn_decode_splitk_bias.restype = i32
    L.attn_splitk_merge_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, vp]
    L.attn_splitk_merge_backward.restype = i32
    L.attn_decode_splitk_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                             f32, i32, i32, vp]
    L.attn_decode_splitk_noalloc.restype = i32
    L.attn_decode_workspace_bytes_multi.argtypes = [i32, i32, i32, i32, i32]
    L.attn_decode_workspace_bytes_multi.restype = sz
    L.attn_decode_splitk_multi.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                           i32, f32, i32, vp, sz, i32, vp]
    L.attn_decode_splitk_multi.restype = i32
    L.attn_decode_splitk_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                         i32, f32, i32, vp, sz, i32, vp]
    L.attn_decode_splitk_fp8.restype = i32
    L.gqa_ceiling_mfma_flops.argtypes = [i32, i32]
    L.gqa_ceiling_mfma_flops.restype = ctypes.c_longlong
    L.gqa_ceiling_mfma.argtypes = [i32, i32, vp, vp]
    L.gqa_ceiling_mfma.restype = i32
    L.gqa_ceiling_stream_read.argtypes = [vp, sz, i32, vp, vp]
    L.gqa_ceiling_stream_read.restype = i32
    L.attn_status_str.argtypes = [i32]
    L.attn_status_str.restype = ctypes.c_char_p
    _lib = L
    return L


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(fn: str, rc: int):
    if rc != 0:
        raise GqaError(fn, rc)


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


# ---- argument checks: a tensor the kernels would read or write out of bounds
# (wrong shape, device or layout) is refused here, before any launch ----------

def _gpu_contig(name: str, t: torch.Tensor, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _int32_table(name: str, t: torch.Tensor, device):
    _gpu_contig(name, t, device)
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be an int32 tensor")


def _out_tensor(name: str, t: Optional[torch.Tensor], shape, dtype, device) -> torch.Tensor:
    """A caller-given output must have exactly the shape and dtype the kernels write."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _gpu_contig(name, t, device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    return t


def _kernel_code(kernel) -> int:
    if kernel not in PREFILL_KERNELS:
        raise ValueError(f"kernel must be one of {sorted(k for k in PREFILL_KERNELS if k)} or None")
    return PREFILL_KERNELS[kernel]


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True,
             scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
             lse: Optional[torch.Tensor] = None, kv_splits: Optional[int] = None,
             kernel: Optional[str] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention forward. q [B,Hq,q_len,D], k/v [B,Hkv,kv_len,D] on one GPU.

    Returns (o [B,Hq,q_len,D] in q's dtype, lse [B,Hq,q_len] fp32, natural log).
    Causal masking is bottom-right aligned (query i sees keys j <= i + kv_len - q_len).
    kv_splits: key ranges per block of query rows (attn_fwd_split); None lets the
    library choose (attn_fwd_kv_splits), 1 forces the single-pass forward.
    kernel: None / "auto" (by shape), "pingpong" or "fourwave" (bf16 / fp16
    single pass; for tests that cover both kernels).
    """
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k/v must be 4-D: [B, H, len, D]")
    B, Hq, q_len, D = q.shape
    Bk, Hkv, kv_len, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch between q, k and v")
    if q.dtype not in _TORCH_DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype among float32/float16/bfloat16")
    code = _kernel_code(kernel)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _gpu_contig(name, t, q.device)
    out = _out_tensor("out", out, q.shape, q.dtype, q.device)
    lse = _out_tensor("lse", lse, (B, Hq, q_len), torch.float32, q.device)
    sc = default_scale(D) if scale is None else float(scale)
    dt = _TORCH_DT[q.dtype]
    if kv_splits is None:
        kv_splits = 1 if code else int(lib().attn_fwd_kv_splits(B, Hq, Hkv, q_len, kv_len, D,
                                                                 int(bool(causal)), dt))
    if kv_splits > 1:
        # small grids: key ranges in parallel, merged by LSE (workspace from torch's allocator)
        ws = torch.empty(int(lib().attn_fwd_split_workspace_bytes(B, Hq, q_len, D, kv_splits)),
                         dtype=torch.uint8, device=q.device)
        rc = lib().attn_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, q_len, kv_len, D,
                                  sc, int(bool(causal)), int(kv_splits), _ptr(ws), ws.numel(), dt,
                                  _stream(q.device))
        _check("attn_fwd_split", rc)
        return out, lse
    if code:
        rc = lib().attn_fwd_with_kernel(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, q_len,
                                        kv_len, D, sc, int(bool(causal)), dt, code, _stream(q.device))
        _check("attn_fwd_with_kernel", rc)
        return out, lse
    rc = lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, q_len, kv_len, D,
                        sc, int(bool(causal)), dt, _stream(q.device))
    _check("attn_fwd", rc)
    return out, lse


def _bias_strides(bias: torch.Tensor, shape) -> Tuple[int, int, int]:
    """Element strides (b, h, i) of a bias broadcast to `shape` = (B, H, rows,
    keys); its last dimension must be contiguous."""
    if bias.dim() != 4:
        raise ValueError("bias must be 4-D, broadcastable to " + str(tuple(shape)))
    try:
        full = bias.expand(*shape)
    except RuntimeError as e:
        raise ValueError(f"bias {tuple(bias.shape)} does not broadcast to {tuple(shape)}") from e
    if shape[3] > 1 and full.stride(3) != 1:
        raise ValueError("the bias must be contiguous along the keys")
    return full.stride(0), full.stride(1), full.stride(2)


def attn_fwd_bias(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, bias: torch.Tensor, causal: bool = False,
                  scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention forward with an additive bias (natural units) added to the
    scaled scores.  q [B,Hq,q_len,D], k/v [B,Hkv,kv_len,D] (fp16 / bf16); bias in
    q's dtype, broadcastable to [B, Hq, q_len, kv_len] (size-1 dimensions are
    read with stride 0), keys contiguous.  Returns (o, lse) as attn_fwd."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k/v must be 4-D: [B, H, len, D]")
    B, Hq, q_len, D = q.shape
    Bk, Hkv, kv_len, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch between q, k and v")
    if q.dtype not in (torch.float16, torch.bfloat16) or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype, float16 or bfloat16")
    if bias.dtype != q.dtype:
        raise TypeError("the bias must have q's dtype")
    sb, sh, sq = _bias_strides(bias, (B, Hq, q_len, kv_len))
    for name, t in (("q", q), ("k", k), ("v", v)):
        _gpu_contig(name, t, q.device)
    if not bias.is_cuda or bias.device != q.device:
        raise ValueError("the bias must be on q's GPU")
    out = _out_tensor("out", out, q.shape, q.dtype, q.device)
    lse = _out_tensor("lse", lse, (B, Hq, q_len), torch.float32, q.device)
    sc = default_scale(D) if scale is None else float(scale)
    rc = lib().attn_fwd_bias(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), sb, sh, sq, _ptr(out), _ptr(lse), B, Hq, Hkv,
                             q_len, kv_len, D, sc, int(bool(causal)), _TORCH_DT[q.dtype], _stream(q.device))
    _check("attn_fwd_bias", rc)
    return out, lse


def attn_prefill_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       qo_indptr: torch.Tensor, kv_indptr: torch.Tensor, kv_indices: torch.Tensor,
                       max_q_len: int, kv_last_page_len: Optional[torch.Tensor] = None, causal: bool = True,
                       scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None,
                       kernel: Optional[str] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Prefill of a batch of ragged requests over a paged KV cache.

    q [total_q, Hq, D] token-major; k/v_cache [num_pages, page_size, Hkv, D];
    qo_indptr, kv_indptr [B+1] int32; kv_indices int32 page ids; optional
    kv_last_page_len [B] int32.  `max_q_len` (a host int) must bound every
    request's query count.  Returns (o [total_q, Hq, D], lse [total_q, Hq] fp32).
    kernel: None / "auto", "pingpong" or "fourwave" (as for attn_fwd).
    """
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [total_q, Hq, D] and the pool [num_pages, page_size, Hkv, D]")
    total_q, Hq, D = q.shape
    _, page_size, Hkv, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between q and the K/V pool")
    if q.dtype not in _TORCH_DT or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and the K/V pool must share one dtype")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _gpu_contig(name, t, q.device)
    for name, t in (("qo_indptr", qo_indptr), ("kv_indptr", kv_indptr), ("kv_indices", kv_indices)) + \
            (() if kv_last_page_len is None else (("kv_last_page_len", kv_last_page_len),)):
        _int32_table(name, t, q.device)
    B = qo_indptr.numel() - 1
    if kv_indptr.numel() != B + 1 or (kv_last_page_len is not None and kv_last_page_len.numel() != B):
        raise ValueError("qo_indptr and kv_indptr need B + 1 entries, kv_last_page_len B")
    code = _kernel_code(kernel)
    if check_tables:
        check_paged_prefill_tables(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, k_cache.shape[0],
                                   page_size, int(max_q_len), total_q)
    out = _out_tensor("out", out, q.shape, q.dtype, q.device)
    lse = _out_tensor("lse", lse, (total_q, Hq), torch.float32, q.device)
    sc = default_scale(D) if scale is None else float(scale)
    rc = lib().attn_prefill_paged_with_kernel(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                                              _ptr(qo_indptr), _ptr(kv_indptr), _ptr(kv_indices),
                                              _ptr(kv_last_page_len), B, Hq, Hkv, D, page_size, int(max_q_len),
                                              sc, int(bool(causal)), _TORCH_DT[q.dtype], code, _stream(q.device))
    _check("attn_prefill_paged", rc)
    return out, lse


# ---- host-side checks of the tables the kernels trust --------------------------
# The kernels read sequence lengths, block tables and CSR pointers without
# bounds checks (an out-of-range page id is undefined behaviour).  These checks
# copy the tables to the host (a synchronising copy) and raise ValueError at the
# first entry a kernel would read out of range.  They run before every launch
# when `check_tables` is true (set from GQA_ATTN_CHECK_TABLES=1 when the module
# is imported, or by set_check_tables), and can be called directly.

def _host_ints(t: torch.Tensor):
    return t.detach().to("cpu", torch.int64).reshape(-1).tolist()


def check_decode_tables(seq_lens: torch.Tensor, block_table: Optional[torch.Tensor], page_size: int,
                        num_pages: int, max_kv_len: int) -> None:
    """seq_lens [B]: 0 <= len <= max_kv_len.  block_table [B, max_pages] (paged):
    the ceil(len / page_size) entries of row b that the kernels read lie in
    [0, num_pages) and fit the row."""
    lens = _host_ints(seq_lens)
    for b, n in enumerate(lens):
        if n < 0 or n > max_kv_len:
            raise ValueError(f"seq_lens[{b}] = {n} outside [0, {max_kv_len}]")
    if block_table is None:
        return
    max_pages = block_table.shape[1]
    rows = block_table.detach().to("cpu", torch.int64)
    for b, n in enumerate(lens):
        used = (n + page_size - 1) // page_size
        if used > max_pages:
            raise ValueError(f"sequence {b} needs {used} pages, the block table has {max_pages} per row")
        for j, pg in enumerate(rows[b, :used].tolist()):
            if pg < 0 or pg >= num_pages:
                raise ValueError(f"block_table[{b}, {j}] = {pg} outside [0, {num_pages})")


def check_paged_prefill_tables(qo_indptr: torch.Tensor, kv_indptr: torch.Tensor, kv_indices: torch.Tensor,
                               kv_last_page_len: Optional[torch.Tensor], num_pages: int, page_size: int,
                               max_q_len: int, total_q: int) -> None:
    """CSR pointers non-decreasing from 0, within their arrays; every request's
    query count <= max_q_len; page ids in [0, num_pages); a request with pages
    has 1 <= kv_last_page_len <= page_size."""
    qo, kvp, idx = _host_ints(qo_indptr), _host_ints(kv_indptr), _host_ints(kv_indices)
    B = len(qo) - 1
    if len(kvp) != B + 1:
        raise ValueError("qo_indptr and kv_indptr must have the same length")
    if qo[0] != 0 or kvp[0] != 0:
        raise ValueError("qo_indptr[0] and kv_indptr[0] must be 0")
    if qo[-1] > total_q or kvp[-1] > len(idx):
        raise ValueError("the pointers run past q or kv_indices")
    last = None if kv_last_page_len is None else _host_ints(kv_last_page_len)
    for b in range(B):
        nq, npg = qo[b + 1] - qo[b], kvp[b + 1] - kvp[b]
        if nq < 0 or npg < 0:
            raise ValueError(f"request {b}: decreasing pointers")
        if nq > max_q_len:
            raise ValueError(f"request {b}: {nq} queries > max_q_len = {max_q_len}")
        if npg > 0 and last is not None and not 1 <= last[b] <= page_size:
            raise ValueError(f"kv_last_page_len[{b}] = {last[b]} outside [1, {page_size}]")
    for j, pg in enumerate(idx[:kvp[-1]]):
        if pg < 0 or pg >= num_pages:
            raise ValueError(f"kv_indices[{j}] = {pg} outside [0, {num_pages})")


check_tables = os.environ.get("GQA_ATTN_CHECK_TABLES") == "1"


def set_check_tables(on: bool) -> None:
    """Check (or stop checking) every table on the host before each launch."""
    global check_tables
    check_tables = bool(on)


def decode_workspace_bytes(B: int, Hq: int, D: int, n_splits: int) -> int:
    return int(lib().attn_decode_workspace_bytes(B, Hq, D, n_splits))


def _decode_geometry(q, k, v, seq_lens, block_table, max_kv_len, kv_dtype):
    """Shapes of a decode call, checked against each other: q [B, Hq, (q_len,) D];
    paged k/v [pages, page_size, Hkv, D] with block_table [B, max_pages], or dense
    k/v [B, Hkv, L, D] (then max_kv_len, the row stride in tokens, must be L);
    seq_lens [B].  Returns (Hkv, page_size, max_pages, max_kv_len)."""
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("q must be bfloat16 or float16")
    if k.dtype != kv_dtype or v.dtype != kv_dtype:
        raise TypeError(f"k and v must be {kv_dtype}")
    if k.dim() != 4 or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be 4-D tensors of one shape")
    B, D = q.shape[0], q.shape[-1]
    if k.shape[3] != D:
        raise ValueError(f"head dim of k ({k.shape[3]}) differs from q's ({D})")
    if seq_lens.numel() != B:
        raise ValueError(f"seq_lens has {seq_lens.numel()} entries for a batch of {B}")
    if block_table is not None:
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise ValueError("block_table must be [B, max_pages]")
        _, page_size, Hkv, _ = k.shape
        max_pages = block_table.shape[1]
        if max_kv_len is None:
            max_kv_len = max_pages * page_size
        if not 0 <= int(max_kv_len) <= max_pages * page_size:
            raise ValueError("max_kv_len must be within the block table's max_pages * page_size keys")
    else:
        Bk, Hkv, L, _ = k.shape
        if Bk != B:
            raise ValueError(f"dense k/v hold {Bk} sequences for a batch of {B}")
        page_size, max_pages = 0, 0
        if max_kv_len is None:
            max_kv_len = L
        if int(max_kv_len) != L:
            raise ValueError(f"dense layout: max_kv_len ({max_kv_len}) must equal k.shape[2] ({L}), "
                             "the row stride in tokens")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _gpu_contig(name, t, q.device)
    _int32_table("seq_lens", seq_lens, q.device)
    if block_table is not None:
        _int32_table("block_table", block_table, q.device)
    return Hkv, page_size, max_pages, int(max_kv_len)


def _workspace(ws: Optional[torch.Tensor], need: int, device) -> torch.Tensor:
    if ws is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    _gpu_contig("workspace", ws, device)
    return ws


def attn_decode_splitk(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor,
                       block_table: Optional[torch.Tensor] = None, n_splits: int = 16,
                       scale: Optional[float] = None, max_kv_len: Optional[int] = None,
                       workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-K decode. q [B,Hq,D]; paged k/v [pages,page_size,Hkv,D] with block_table
    [B,max_pages] int32, or dense k/v [B,Hkv,max_kv_len,D] with block_table None.

    Returns (o [B,Hq,D], lse [B,Hq] fp32).  `workspace` (uint8, >= decode_workspace_bytes)
    may be passed to avoid an allocation per call.
    """
    if q.dim() != 3:
        raise ValueError("q must be [B, Hq, D]")
    B, Hq, D = q.shape
    Hkv, page_size, max_pages, max_kv_len = _decode_geometry(q, k, v, seq_lens, block_table, max_kv_len, q.dtype)
    if check_tables:
        check_decode_tables(seq_lens, block_table, page_size, k.shape[0], max_kv_len)
    workspace = _workspace(workspace, decode_workspace_bytes(B, Hq, D, n_splits), q.device)
    out = _out_tensor("out", out, q.shape, q.dtype, q.device)
    lse = _out_tensor("lse", lse, (B, Hq), torch.float32, q.device)
    sc = default_scale(D) if scale is None else float(scale)
    rc = lib().attn_decode_splitk(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(seq_lens),
                                  _ptr(block_table), max_pages, page_size, B, Hq, Hkv, D,
                                  max_kv_len, sc, int(n_splits), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  _TORCH_DT[q.dtype], _stream(q.device))
    _check("attn_decode_splitk", rc)
    return out, lse


def attn_decode_splitk_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor,
                               out: torch.Tensor, lse: torch.Tensor, block_table: Optional[torch.Tensor] = None,
                               n_splits: int = 16, scale: Optional[float] = None,
                               max_kv_len: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """attn_decode_splitk with the library's fixed device scratch instead of a
    workspace: nothing is allocated, so `out` [B,Hq,D] and `lse` [B,Hq] fp32
    must be given.  Calls that overlap on one GPU race on the scratch."""
    if q.dim() != 3:
        raise ValueError("q must be [B, Hq, D]")
    B, Hq, D = q.shape
    Hkv, page_size, max_pages, max_kv_len = _decode_geometry(q, k, v, seq_lens, block_table, max_kv_len, q.dtype)
    if check_tables:
        check_decode_tables(seq_lens, block_table, page_size, k.shape[0], max_kv_len)
    if out is None or lse is None:
        raise ValueError("out and lse must be given (this call allocates nothing)")
    out = _out_tensor("out", out, q.shape, q.dtype, q.device)
    lse = _out_tensor("lse", lse, (B, Hq), torch.float32, q.device)
    sc = default_scale(D) if scale is None else float(scale)
    rc = lib().attn_decode_splitk_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(seq_lens),
                                          _ptr(block_table), max_pages, page_size, B, Hq, Hkv, D, max_kv_len, sc,
                                          int(n_splits), _TORCH_DT[q.dtype], _stream(q.device))
    _check("attn_decode_splitk_noalloc", rc)
    return out, lse


def attn_decode_splitk_fp8(q: torch.Tensor, k8: torch.Tensor, v8: torch.Tensor, k_scale_shift: torch.Tensor,
                           v_scale_shift: torch.Tensor, seq_lens: torch.Tensor,
                           block_table: Optional[torch.Tensor] = None, n_splits: int = 16,
                           scale: Optional[float] = None, max_kv_len: Optional[int] = None,
                           workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-K decode over an E4M3 KV cache. q [B,Hq,D] bf16/fp16; k8/v8 uint8
    [pages,page_size,Hkv,D] with block_table (page_size >= 16) or [B,Hkv,max_kv_len,D];
    k/v_scale_shift int32 [pages,page_size,Hkv] or [B,Hkv,max_kv_len] (binary16
    scale in bits 0-15, shift in bits 16-31).  Returns (o [B,Hq,D], lse [B,Hq])."""
    if q.dim() != 3:
        raise ValueError("q must be [B, Hq, D]")
    B, Hq, D = q.shape
    Hkv, page_size, max_pages, max_kv_len = _decode_geometry(q, k8, v8, seq_lens, block_table, max_kv_len,
                                                             torch.uint8)
    for name, t in (("k_scale_shift", k_scale_shift), ("v_scale_shift", v_scale_shift)):
        if tuple(t.shape) != tuple(k8.shape[:3]):
            raise ValueError(f"{name} must be {tuple(k8.shape[:3])} (one word per token row and head)")
        _int32_table(name, t, q.device)
    if check_tables:
        check_decode_tables(seq_lens, block_table, page_size, k8.shape[0], max_kv_len)
    workspace = _workspace(workspace, decode_workspace_bytes(B, Hq, D, n_splits), q.device)
    out = _out_tensor("out", out, q.shape, q.dtype, q.device)
    lse = _out_tensor("lse", lse, (B, Hq), torch.float32, q.device)
    sc = default_scale(D) if scale is None else float(scale)
    rc = lib().attn_decode_splitk_fp8(_ptr(q), _ptr(k8), _ptr(v8), _ptr(k_scale_shift), _ptr(v_scale_shift),
                                      _ptr(out), _ptr(lse), _ptr(seq_lens), _ptr(block_table), max_pages,
                                      page_size, B, Hq, Hkv, D, max_kv_len, sc, int(n_splits), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _TORCH_DT[q.dtype],
                                      _stream(q.device))
    _check("attn_decode_splitk_fp8", rc)
    return out, lse


def decode_workspace_bytes_multi(B: int, Hq: int, q_len: int, D: int, n_splits: int) -> int:
    return int(lib().attn_decode_workspace_bytes_multi(B, Hq, q_len, D, n_splits))


def attn_decode_splitk_multi(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor,
                             block_table: Optional[torch.Tensor] = None, n_splits: int = 16,
                             scale: Optional[float] = None, max_kv_len: Optional[int] = None,
                             workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                             lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-K decode of q_len queries per sequence at its last positions (causal
    among themselves: query i sees keys t <= seq_lens[b] - q_len + i).

    q [B,Hq,q_len,D]; k/v and block_table as for attn_decode_splitk.
    Returns (o [B,Hq,q_len,D], lse [B,Hq,q_len] fp32).
    """
    if q.dim() != 4:
        raise ValueError("q must be [B, Hq, q_len, D]")
    B, Hq, q_len, D = q.shape
    Hkv, page_size, max_pages, max_kv_len = _decode_geometry(q, k, v, seq_lens, block_table, max_kv_len, q.dtype)
    if check_tables:
        check_decode_tables(seq_lens, block_table, page_size, k.shape[0], max_kv_len)
    workspace = _workspace(workspace, decode_workspace_bytes_multi(B, Hq, q_len, D, n_splits), q.device)
    out = _out_tensor("out", out, q.shape, q.dtype, q.device)
    lse = _out_tensor("lse", lse, (B, Hq, q_len), torch.float32, q.device)
    sc = default_scale(D) if scale is None else float(scale)
    rc = lib().attn_decode_splitk_multi(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(seq_lens),
                                        _ptr(block_table), max_pages, page_size, B, Hq, Hkv, q_len, D,
                                        max_kv_len, sc, int(n_splits), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _TORCH_DT[q.dtype], _stream(q.device))
    _check("attn_decode_splitk_multi", rc)
    return out, lse


# ---- measurement kernels (include/gqa_ceilings.h) ----------------------------

def ceiling_mfma(n_workgroups: int, iters: int, out: Optional[torch.Tensor] = None) -> Tuple[int, torch.Tensor]:
    """Launch the MFMA-only loop on the current stream; returns (flops of the
    launch, its output buffer)."""
    dev = torch.device("cuda", torch.cuda.current_device())
    out = _out_tensor("out", out, (n_workgroups * 512,), torch.float32, dev)
    rc = lib().gqa_ceiling_mfma(int(n_workgroups), int(iters), _ptr(out), _stream(dev))
    if rc:
        raise RuntimeError(f"gqa_ceiling_mfma failed ({rc})")
    return int(lib().gqa_ceiling_mfma_flops(int(n_workgroups), int(iters))), out


def ceiling_stream_read(src: torch.Tensor, n_workgroups: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Read every byte of `src` (a contiguous GPU tensor) once on the current stream."""
    _gpu_contig("src", src)
    out = _out_tensor("out", out, (n_workgroups,), torch.int32, src.device)
    rc = lib().gqa_ceiling_stream_read(_ptr(src), src.numel() * src.element_size(), int(n_workgroups), _ptr(out),
                                       _stream(src.device))
    if rc:
        raise RuntimeError(f"gqa_ceiling_stream_read failed ({rc})")
    return out


def attn_decode_splitk_bias(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor,
                            bias: torch.Tensor, block_table: Optional[torch.Tensor] = None, n_splits: int = 16,
                            scale: Optional[float] = None, max_kv_len: Optional[int] = None,
                            workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-K decode of q_len queries per sequence (q [B,Hq,q_len,D], as
    attn_decode_splitk_multi) with an additive bias: query i of sequence b,
    head h, key t gets bias[b, h, i, t] (natural units, q's dtype).  bias is
    broadcastable to [B, Hq, q_len, L] with L >= every sequence length, keys
    contiguous, even strides; rows of an odd length need one readable element
    past it.  Returns (o [B,Hq,q_len,D], lse [B,Hq,q_len] fp32)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, Hq, q_len, D]")
    B, Hq, q_len, D = q.shape
    Hkv, page_size, max_pages, max_kv_len = _decode_geometry(q, k, v, seq_lens, block_table, max_kv_len, q.dtype)
    if bias.dtype != q.dtype:
        raise TypeError("the bias must have q's dtype")
    sb, sh, sq = _bias_strides(bias, (B, Hq, q_len, bias.shape[-1]))
    if (sb | sh | sq) & 1 or bias.data_ptr() % 4:
        raise ValueError("the bias needs even strides and a 4-byte aligned start (keys are read in pairs)")
    if not bias.is_cuda or bias.device != q.device:
        raise ValueError("the bias must be on q's GPU")
    if check_tables:
        check_decode_tables(seq_lens, block_table, page_size, k.shape[0], max_kv_len)
        if int(seq_lens.max()) > bias.shape[-1]:
            raise ValueError("the bias has fewer keys than a sequence")
    workspace = _workspace(workspace, decode_workspace_bytes_multi(B, Hq, q_len, D, n_splits), q.device)
    out = _out_tensor("out", out, q.shape, q.dtype, q.device)
    lse = _out_tensor("lse", lse, (B, Hq, q_len), torch.float32, q.device)
    sc = default_scale(D) if scale is None else float(scale)
    rc = lib().attn_decode_splitk_bias(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), sb, sh, sq, _ptr(out), _ptr(lse),
                                       _ptr(seq_lens), _ptr(block_table), max_pages, page_size, B, Hq, Hkv, q_len, D,
                                       max_kv_len, sc, int(n_splits), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _TORCH_DT[q.dtype],
                                       _stream(q.device))
    _check("attn_decode_splitk_bias", rc)
    return out, lse


def attn_splitk_merge_backward(o_parts: torch.Tensor, lse_parts: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
                               d_o: torch.Tensor, d_lse: torch.Tensor, d_o_parts: Optional[torch.Tensor] = None,
                               d_lse_parts: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Gradients of the split-K merge with respect to its partials (fp32):
    o_parts [..., S, D], lse_parts [..., S], o / d_o [..., D], lse / d_lse [...].
    Returns (d_o_parts [..., S, D], d_lse_parts [..., S])."""
    if o_parts.dim() < 2:
        raise ValueError("o_parts must be [..., n_splits, D]")
    S, D = o_parts.shape[-2], o_parts.shape[-1]
    lead = tuple(o_parts.shape[:-2])
    want = {"lse_parts": (lse_parts, lead + (S,)), "o": (o, lead + (D,)), "lse": (lse, lead),
            "d_o": (d_o, lead + (D,)), "d_lse": (d_lse, lead)}
    for name, (t, shape) in want.items():
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must be {shape}, got {tuple(t.shape)}")
    for name, t in [("o_parts", o_parts)] + [(n, t) for n, (t, _) in want.items()]:
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
        _gpu_contig(name, t, o_parts.device)
    d_o_parts = _out_tensor("d_o_parts", d_o_parts, o_parts.shape, torch.float32, o_parts.device)
    d_lse_parts = _out_tensor("d_lse_parts", d_lse_parts, lse_parts.shape, torch.float32, o_parts.device)
    rows = int(math.prod(lead)) if lead else 1
    rc = lib().attn_splitk_merge_backward(_ptr(o_parts), _ptr(lse_parts), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(d_lse),
                                          _ptr(d_o_parts), _ptr(d_lse_parts), rows, S, D, _stream(o_parts.device))
    _check("attn_splitk_merge_backward", rc)
    return d_o_parts, d_lse_parts
