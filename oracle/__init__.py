"""fp64 CPU oracle for GQA attention forward and split-K paged decode.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this package; the HIP library and its Python
binding never do, and this package never imports them.

The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over query rows);
this module only marshals torch CPU tensors into it and returns numpy float64
arrays.  Which passages of the pages each function follows is stated in the C
source next to each function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
# The mutation tests point this at a deliberately broken build of oracle.c.
_LIB_OVERRIDE = os.environ.get("GQA_ORACLE_LIB")

_DT = {torch.float64: 0, torch.float32: 1, torch.float16: 2, torch.bfloat16: 3}
FP8_E4M3 = 4  # storage code of an 8-bit E4M3 cache given as uint8 bytes

_lib = None


def build(src: str = _SRC, out: str = LIB_PATH) -> str:
    """Compile oracle.c (or a given copy of it) into a shared library with gcc."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-Wextra", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_widen.argtypes = [vp, i32, i64, vp]
    lib.oracle_widen.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    lib.oracle_attn_fwd.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    f64, i32, vp, i64, vp, vp]
    lib.oracle_attn_fwd.restype = i32
    lib.oracle_softmax_matrix.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                          f64, i32, i32, i32, vp]
    lib.oracle_softmax_matrix.restype = i32
    lib.oracle_attn_decode.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                       i32, i32, f64, vp, i64, vp, vp]
    lib.oracle_attn_decode.restype = i32
    lib.oracle_decode_split_merge.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32,
                                              i32, i32, i32, f64, vp, i32, vp, i64, vp, vp,
                                              vp, vp]
    lib.oracle_decode_split_merge.restype = i32
    lib.oracle_attn_decode_multi.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                             i32, i32, i32, f64, vp, i64, vp, vp]
    lib.oracle_attn_decode_multi.restype = i32
    lib.oracle_attn_prefill_paged.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32,
                                              i32, f64, i32, vp, i64, vp, vp]
    lib.oracle_attn_prefill_paged.restype = i32
    lib.oracle_attn_decode_fp8.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                           i32, f64, vp, i64, vp, vp]
    lib.oracle_attn_decode_fp8.restype = i32
    lib.oracle_attn_fwd_bias.argtypes = [vp, vp, vp, i32, vp, i32, i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                         f64, i32, vp, i64, vp, vp]
    lib.oracle_attn_fwd_bias.restype = i32
    lib.oracle_attn_decode_bias.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                            f64, vp, i32, i64, i64, i64, vp, i64, vp, vp]
    lib.oracle_attn_decode_bias.restype = i32
    lib.oracle_splitk_merge.argtypes = [vp, vp, i64, i32, i32, vp, vp]
    lib.oracle_splitk_merge.restype = i32
    lib.oracle_splitk_merge_backward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i32, i32, vp, vp]
    lib.oracle_splitk_merge_backward.restype = i32
    _lib = lib
    return lib


def num_threads() -> int:
    """OpenMP threads the oracle runs on."""
    return int(_load().oracle_num_threads())


def _cpu(t: torch.Tensor, dtype=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        t = torch.as_tensor(t)
    t = t.detach().to("cpu")
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _np_ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _dt(*ts):
    dts = {t.dtype for t in ts}
    if len(dts) != 1:
        raise TypeError(f"q/k/v must share one dtype, got {dts}")
    dt = dts.pop()
    if dt not in _DT:
        raise TypeError(f"unsupported dtype {dt}")
    return _DT[dt]


def _rows(rows):
    if rows is None:
        return None
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r


def widen(t: torch.Tensor, fp8: bool = False) -> np.ndarray:
    """The oracle's own storage-format -> float64 conversion (for pinning it);
    fp8=True reads a uint8 tensor as E4M3 bytes."""
    t = _cpu(t)
    out = np.empty(t.numel(), dtype=np.float64)
    code = FP8_E4M3 if fp8 else _DT[t.dtype]
    _load().oracle_widen(_ptr(t), code, t.numel(), _np_ptr(out))
    return out.reshape(tuple(t.shape))


def attn_fwd(q, k, v, scale: float, causal: bool, rows=None):
    """Plain attention forward.

    q [B, Hq, q_len, D], k/v [B, Hkv, kv_len, D] (one storage dtype).
    Returns (o, lse): with rows=None, o [B, Hq, q_len, D] and lse [B, Hq, q_len];
    otherwise o [n, D] and lse [n] for the flat row ids (b*Hq + h)*q_len + i.
    `scale` is used exactly as given (pass the fp32 value the GPU receives).
    """
    q, k, v = _cpu(q), _cpu(k), _cpu(v)
    dt = _dt(q, k, v)
    B, Hq, q_len, D = q.shape
    _, Hkv, kv_len, _ = k.shape
    r = _rows(rows)
    n = B * Hq * q_len if r is None else r.shape[0]
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load().oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), dt, B, Hq, Hkv, q_len, kv_len, D,
                                 float(scale), int(bool(causal)), _np_ptr(r), n,
                                 _np_ptr(o), _np_ptr(lse))
    if rc:
        raise ValueError("oracle_attn_fwd: bad arguments")
    if r is None:
        return o.reshape(B, Hq, q_len, D), lse.reshape(B, Hq, q_len)
    return o, lse


def softmax_matrix(q, k, scale: float, causal: bool, b: int, h: int) -> np.ndarray:
    """Materialised softmax P [q_len, kv_len] of one (b, h)."""
    q, k = _cpu(q), _cpu(k)
    dt = _dt(q, k)
    B, Hq, q_len, D = q.shape
    _, Hkv, kv_len, _ = k.shape
    p = np.empty((q_len, kv_len), dtype=np.float64)
    rc = _load().oracle_softmax_matrix(_ptr(q), _ptr(k), dt, B, Hq, Hkv, q_len, kv_len, D,
                                       float(scale), int(bool(causal)), b, h, _np_ptr(p))
    if rc:
        raise ValueError("oracle_softmax_matrix: bad arguments")
    return p


def _decode_common(q, k, v, seq_lens, block_table, max_kv_len):
    q, k, v = _cpu(q), _cpu(k), _cpu(v)
    dt = _dt(q, k, v)
    B, Hq, D = q.shape[0], q.shape[1], q.shape[-1]
    sl = _cpu(seq_lens, torch.int32)
    if block_table is not None:
        bt = _cpu(block_table, torch.int32)
        max_pages = bt.shape[1]
        page_size = k.shape[1]
        Hkv = k.shape[2]
        if max_kv_len is None:
            max_kv_len = max_pages * page_size
    else:
        bt = None
        max_pages, page_size = 0, 0
        Hkv = k.shape[1]
        if max_kv_len is None:
            max_kv_len = k.shape[2]
    return q, k, v, dt, B, Hq, D, sl, bt, max_pages, page_size, Hkv, int(max_kv_len)


def attn_decode(q, k, v, seq_lens, scale: float, block_table=None, max_kv_len=None, rows=None):
    """Decode (q_len = 1) over a paged pool (block_table given) or dense [B, Hkv, L, D] K/V.

    Returns (o [B, Hq, D], lse [B, Hq]) or, with rows, (o [n, D], lse [n]) for
    flat ids b*Hq + h.
    """
    q, k, v, dt, B, Hq, D, sl, bt, max_pages, page_size, Hkv, max_kv_len = _decode_common(
        q, k, v, seq_lens, block_table, max_kv_len)
    r = _rows(rows)
    n = B * Hq if r is None else r.shape[0]
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load().oracle_attn_decode(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(sl), _ptr(bt), max_pages,
                                    page_size, B, Hq, Hkv, D, max_kv_len, float(scale),
                                    _np_ptr(r), n, _np_ptr(o), _np_ptr(lse))
    if rc:
        raise ValueError("oracle_attn_decode: bad arguments")
    if r is None:
        return o.reshape(B, Hq, D), lse.reshape(B, Hq)
    return o, lse


def decode_split_merge(q, k, v, seq_lens, scale: float, bounds, block_table=None,
                       max_kv_len=None, rows=None):
    """Decode computed chunk by chunk and merged through the chunks' LSEs.

    bounds: int array [B, n_splits + 1] of chunk edges per sequence.
    Returns (o, lse, o_parts, lse_parts) with o [n, D], lse [n],
    o_parts [n, n_splits, D], lse_parts [n, n_splits] over flat ids b*Hq + h.
    """
    q, k, v, dt, B, Hq, D, sl, bt, max_pages, page_size, Hkv, max_kv_len = _decode_common(
        q, k, v, seq_lens, block_table, max_kv_len)
    bnd = _cpu(torch.as_tensor(bounds), torch.int32)
    n_splits = bnd.shape[1] - 1
    r = _rows(rows)
    n = B * Hq if r is None else r.shape[0]
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    op = np.empty((n, n_splits, D), dtype=np.float64)
    lp = np.empty((n, n_splits), dtype=np.float64)
    rc = _load().oracle_decode_split_merge(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(sl), _ptr(bt),
                                           max_pages, page_size, B, Hq, Hkv, D, max_kv_len,
                                           float(scale), _ptr(bnd), n_splits, _np_ptr(r), n,
                                           _np_ptr(o), _np_ptr(lse), _np_ptr(op), _np_ptr(lp))
    if rc:
        raise ValueError("oracle_decode_split_merge: bad arguments")
    return o, lse, op, lp


def attn_decode_multi(q, k, v, seq_lens, scale: float, block_table=None, max_kv_len=None, rows=None):
    """Decode of q_len queries per sequence, placed at its last q_len positions
    (query i sees keys t <= seq_lens[b] - q_len + i).

    q [B, Hq, q_len, D]; K/V as for attn_decode.  Returns (o [B, Hq, q_len, D],
    lse [B, Hq, q_len]) or, with rows, (o [n, D], lse [n]) for flat ids
    (b*Hq + h)*q_len + i.
    """
    q, k, v, dt, B, Hq, D, sl, bt, max_pages, page_size, Hkv, max_kv_len = _decode_common(
        q, k, v, seq_lens, block_table, max_kv_len)
    q_len = q.shape[2]
    r = _rows(rows)
    n = B * Hq * q_len if r is None else r.shape[0]
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load().oracle_attn_decode_multi(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(sl), _ptr(bt), max_pages,
                                          page_size, B, Hq, Hkv, q_len, D, max_kv_len, float(scale),
                                          _np_ptr(r), n, _np_ptr(o), _np_ptr(lse))
    if rc:
        raise ValueError("oracle_attn_decode_multi: bad arguments")
    if r is None:
        return o.reshape(B, Hq, q_len, D), lse.reshape(B, Hq, q_len)
    return o, lse


def attn_prefill_paged(q, k_cache, v_cache, qo_indptr, kv_indptr, kv_indices, scale: float,
                       causal: bool = True, kv_last_page_len=None, rows=None):
    """Prefill of ragged requests over a paged KV cache.

    q [total_q, Hq, D] token-major; k/v_cache [num_pages, page_size, Hkv, D];
    qo_indptr, kv_indptr [B + 1] int; kv_indices [nnz_pages] int; optional
    kv_last_page_len [B].  Returns (o [total_q, Hq, D], lse [total_q, Hq]) or,
    with rows, (o [n, D], lse [n]) for flat ids token*Hq + h.
    """
    q, k, v = _cpu(q), _cpu(k_cache), _cpu(v_cache)
    dt = _dt(q, k, v)
    total_q, Hq, D = q.shape
    page_size, Hkv = k.shape[1], k.shape[2]
    qi = _cpu(torch.as_tensor(qo_indptr), torch.int32)
    ki = _cpu(torch.as_tensor(kv_indptr), torch.int32)
    kx = _cpu(torch.as_tensor(kv_indices), torch.int32)
    if kx.numel() == 0:
        kx = torch.zeros(1, dtype=torch.int32)
    last = None if kv_last_page_len is None else _cpu(torch.as_tensor(kv_last_page_len), torch.int32)
    B = qi.numel() - 1
    if int(qi[B]) != total_q:
        raise ValueError("qo_indptr[-1] must equal q.shape[0]")
    r = _rows(rows)
    n = total_q * Hq if r is None else r.shape[0]
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load().oracle_attn_prefill_paged(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(qi), _ptr(ki), _ptr(kx),
                                           _ptr(last), B, Hq, Hkv, D, page_size, float(scale),
                                           int(bool(causal)), _np_ptr(r), n, _np_ptr(o), _np_ptr(lse))
    if rc:
        raise ValueError("oracle_attn_prefill_paged: bad arguments")
    if r is None:
        return o.reshape(total_q, Hq, D), lse.reshape(total_q, Hq)
    return o, lse


def attn_decode_fp8(q, k8, v8, k_ss, v_ss, seq_lens, scale: float, block_table=None, max_kv_len=None,
                    rows=None):
    """Decode over an 8-bit E4M3 KV cache with a binary16 (scale, shift) pair per
    token row and K/V head: the key / value used is byte * scale + shift.

    q [B, Hq, D] (bf16/fp16/fp32); k8, v8 uint8 [num_pages, page_size, Hkv, D]
    (with block_table) or [B, Hkv, max_kv_len, D]; k_ss, v_ss int32/uint32
    [num_pages, page_size, Hkv] or [B, Hkv, max_kv_len] (scale bits 0-15, shift
    bits 16-31).  Returns (o [B, Hq, D], lse [B, Hq]) or, with rows, (o [n, D],
    lse [n]).
    """
    q = _cpu(q)
    if q.dtype not in _DT:
        raise TypeError(f"unsupported q dtype {q.dtype}")
    k8, v8 = _cpu(k8), _cpu(v8)
    if k8.dtype != torch.uint8 or v8.dtype != torch.uint8:
        raise TypeError("the fp8 cache is given as uint8 bytes")
    kss, vss = _cpu(k_ss).view(torch.int32), _cpu(v_ss).view(torch.int32)
    B, Hq, D = q.shape
    sl = _cpu(seq_lens, torch.int32)
    if block_table is not None:
        bt = _cpu(block_table, torch.int32)
        max_pages, page_size, Hkv = bt.shape[1], k8.shape[1], k8.shape[2]
        if max_kv_len is None:
            max_kv_len = max_pages * page_size
    else:
        bt, max_pages, page_size, Hkv = None, 0, 0, k8.shape[1]
        if max_kv_len is None:
            max_kv_len = k8.shape[2]
    r = _rows(rows)
    n = B * Hq if r is None else r.shape[0]
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load().oracle_attn_decode_fp8(_ptr(q), _DT[q.dtype], _ptr(k8), _ptr(v8), _ptr(kss), _ptr(vss),
                                        _ptr(sl), _ptr(bt), max_pages, page_size, B, Hq, Hkv, D,
                                        int(max_kv_len), float(scale), _np_ptr(r), n, _np_ptr(o), _np_ptr(lse))
    if rc:
        raise ValueError("oracle_attn_decode_fp8: bad arguments")
    if r is None:
        return o.reshape(B, Hq, D), lse.reshape(B, Hq)
    return o, lse


def _full_bias(bias, shape) -> torch.Tensor:
    """The bias as a contiguous tensor of the full logical shape (broadcast
    dimensions materialised), in its own storage format."""
    b = torch.as_tensor(bias).detach().to("cpu")
    if b.dtype not in _DT:
        raise TypeError(f"unsupported bias dtype {b.dtype}")
    return b.expand(*shape).contiguous()


def attn_fwd_bias(q, k, v, bias, scale: float, causal: bool, rows=None):
    """Forward with an additive bias: s_ij = scale * q_i.k_j + bias[b, h, i, j].

    bias: a tensor broadcastable to [B, Hq, q_len, kv_len] (any float storage
    format; -inf masks a key).  Other arguments and results as attn_fwd.
    """
    q, k, v = _cpu(q), _cpu(k), _cpu(v)
    dt = _dt(q, k, v)
    B, Hq, q_len, D = q.shape
    _, Hkv, kv_len, _ = k.shape
    bf = _full_bias(bias, (B, Hq, q_len, kv_len))
    r = _rows(rows)
    n = B * Hq * q_len if r is None else r.shape[0]
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = _load().oracle_attn_fwd_bias(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(bf), _DT[bf.dtype],
                                      Hq * q_len * kv_len, q_len * kv_len, kv_len,
                                      B, Hq, Hkv, q_len, kv_len, D, float(scale), int(bool(causal)),
                                      _np_ptr(r), n, _np_ptr(o), _np_ptr(lse))
    if rc:
        raise ValueError("oracle_attn_fwd_bias: bad arguments")
    if r is None:
        return o.reshape(B, Hq, q_len, D), lse.reshape(B, Hq, q_len)
    return o, lse


def attn_decode_bias(q, k, v, seq_lens, bias, scale: float, block_table=None, max_kv_len=None, rows=None):
    """Decode of q_len queries per sequence (as attn_decode_multi; q [B, Hq,
    q_len, D]) with an additive bias: query i of sequence b, head h, key t gets
    bias[b, h, i, t].  bias: broadcastable to [B, Hq, q_len, L] with L >= every
    sequence length.  Returns (o [B, Hq, q_len, D], lse [B, Hq, q_len]) or, with
    rows, (o [n, D], lse [n]) for flat ids (b*Hq + h)*q_len + i."""
    q, k, v, dt, B, Hq, D, sl, bt, max_pages, page_size, Hkv, max_kv_len = _decode_common(
        q, k, v, seq_lens, block_table, max_kv_len)
    q_len = q.shape[2]
    bt_in = torch.as_tensor(bias)
    L = bt_in.shape[-1]
    bf = _full_bias(bt_in, (B, Hq, q_len, L))
    r = _rows(rows)
    n = B * Hq * q_len if r is None else r.shape[0]
    o = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    if sl.numel() and int(sl.max()) > L:
        raise ValueError("the bias has fewer keys than a sequence")
    rc = _load().oracle_attn_decode_bias(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(sl), _ptr(bt), max_pages,
                                         page_size, B, Hq, Hkv, q_len, D, max_kv_len, float(scale),
                                         _ptr(bf), _DT[bf.dtype], Hq * q_len * L, q_len * L, L,
                                         _np_ptr(r), n, _np_ptr(o), _np_ptr(lse))
    if rc:
        raise ValueError("oracle_attn_decode_bias: bad arguments")
    if r is None:
        return o.reshape(B, Hq, q_len, D), lse.reshape(B, Hq, q_len)
    return o, lse


def _f64(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def splitk_merge(o_parts, lse_parts):
    """Merge of partial results: o_parts [..., S, D], lse_parts [..., S] ->
    (o [..., D], lse [...])."""
    op, lp = _f64(o_parts), _f64(lse_parts)
    S, D = op.shape[-2], op.shape[-1]
    lead = lp.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    o = np.empty(lead + (D,), dtype=np.float64)
    lse = np.empty(lead, dtype=np.float64)
    rc = _load().oracle_splitk_merge(_np_ptr(op), _np_ptr(lp), n, S, D, _np_ptr(o), _np_ptr(lse))
    if rc:
        raise ValueError("oracle_splitk_merge: bad arguments")
    return o, lse


def splitk_merge_backward(o_parts, lse_parts, o, lse, d_o, d_lse):
    """Gradients of splitk_merge: given the partials, the merged (o, lse) and
    the gradients (d_o, d_lse) of some scalar with respect to them, returns
    (d_o_parts [..., S, D], d_lse_parts [..., S])."""
    op, lp, oo, ll, do, dl = (_f64(x) for x in (o_parts, lse_parts, o, lse, d_o, d_lse))
    S, D = op.shape[-2], op.shape[-1]
    lead = lp.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    dop = np.empty(op.shape, dtype=np.float64)
    dlp = np.empty(lp.shape, dtype=np.float64)
    rc = _load().oracle_splitk_merge_backward(_np_ptr(op), _np_ptr(lp), _np_ptr(oo), _np_ptr(ll), _np_ptr(do),
                                              _np_ptr(dl), n, S, D, _np_ptr(dop), _np_ptr(dlp))
    if rc:
        raise ValueError("oracle_splitk_merge_backward: bad arguments")
    return dop, dlp
