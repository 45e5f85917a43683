"""CSA / HCA long-context attention for MI355X — thin Python binding of libdsv4attn.so.

Each function marshals torch tensors (device memory, the current HIP stream) into the
C ABI declared in include/dsv4attn.h and returns the output tensors; every step of
the computation runs in the library's HIP kernels.  There is no fallback: if the
library is not built, or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["csa_compress", "csa_compress2", "kv_cache_append", "csa_index_topk", "csa_attend", "hca_attend", "csa_attend_fp8kv",
           "hca_attend_fp8kv", "lse_merge", "lib",
           "LibError",
           "F32", "BF16", "FP8_E4M3", "MXFP4", "FP8_KV", "MXFP4_DTYPE", "FP8_KV_DTYPE", "FP8_ROPE_DIMS"]

F32, BF16, FP8_E4M3, MXFP4, FP8_KV = 0, 1, 2, 3, 4
MXFP4_DTYPE = "mxfp4"            # marker for packed MXFP4 (uint8 codes + uint8 E8M0 scales)
FP8_KV_DTYPE = "fp8_kv"          # marker for FP8 K|V rows (E4M3 codes, bf16 RoPE dims of K)
FP8_ROPE_DIMS = 64               # bf16 tail of an FP8 K row

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsv4attn.so")
# the same library built with -DDSV4_DEBUG (kernel-side checks, see dsv4_debug_flags)
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsv4attn_debug.so")
_lib = None

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_SIGS = {
    "dsv4_version": ([], ctypes.c_int),
    "dsv4_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "dsv4_last_error": ([], ctypes.c_char_p),
    "dsv4_time_next_kernel": ([_p, _p], ctypes.c_int),
    "dsv4_debug_flags": ([ctypes.POINTER(ctypes.c_uint32)], ctypes.c_int),
    "csa_compress": ([_p, ctypes.c_int, _p, _p, _i64, _i64, _i64, _i32, _i64, _p, _p, ctypes.c_int, _i64, _p],
                     ctypes.c_int),
    "csa_compress2": ([_p, _p, ctypes.c_int, _p, _p, _i64, _i64, _i32, _i64, _i64, _p, _p, ctypes.c_int, _i64, _i64,
                       _i64, _p, _p, ctypes.c_int, _i64, _p], ctypes.c_int),
    "kv_cache_append": ([_p, ctypes.c_int, _p, _p, _i64, _i64, _p, _p, _i64, _p, _i32, _p, _p, ctypes.c_int, _i64,
                         _i64, _p], ctypes.c_int),
    "csa_index_topk": ([_p, ctypes.c_int, _p, _p, _p, ctypes.c_int, _p, _i64, _i64, _i32, _i32, _i64, _i64, _i32,
                        _i32, _p, _p, _p, ctypes.POINTER(ctypes.c_size_t), _p], ctypes.c_int),
    "csa_index_topk_noalloc": ([_p, ctypes.c_int, _p, _p, _p, ctypes.c_int, _p, _i64, _i64, _i32, _i32, _i64, _i64,
                                _i32, _i32, _p, _p, _p], ctypes.c_int),
    "csa_attend": ([_p, _p, _p, ctypes.c_int, _p, _i32, _p, _p, _p, _i64, _i32, _p, _i64, _i64, _i32, _i32, _i64,
                    _i64, _i64, _i64, ctypes.c_float, _p, _p, _p, ctypes.POINTER(ctypes.c_size_t), _p], ctypes.c_int),
    "hca_attend": ([_p, _p, _p, ctypes.c_int, _i32, _p, _p, _p, _i64, _i32, _p, _i64, _i64, _i32, _i32, _i64, _i64,
                    _i64, _i64, ctypes.c_float, _p, _p, _p, ctypes.POINTER(ctypes.c_size_t), _p], ctypes.c_int),
    "lse_merge": ([_p, _p, _i32, _i64, _i32, _p, ctypes.c_int, _p, _p], ctypes.c_int),
    "csa_attend_fp8kv": ([_p, _p, _p, _p, _i32, _p, _p, _p, _i64, _i32, _p, _i64, _i64, _i32, _i32, _i32, _i64, _i64,
                          _i64, _i64, ctypes.c_float, ctypes.c_float, ctypes.c_float, _p, _p, _p,
                          ctypes.POINTER(ctypes.c_size_t), _p], ctypes.c_int),
    "hca_attend_fp8kv": ([_p, _p, _p, _i32, _p, _p, _p, _i64, _i32, _p, _i64, _i64, _i32, _i32, _i32, _i64, _i64,
                          _i64, _i64, ctypes.c_float, ctypes.c_float, ctypes.c_float, _p, _p, _p,
                          ctypes.POINTER(ctypes.c_size_t), _p], ctypes.c_int),
}


class BlockPool(ctypes.Structure):
    """dsv4_block_pool: the newest block pooled by csa_pool_index_topk."""
    _fields_ = [("x", _p), ("x2", _p), ("gate", _p), ("pos_bias", _p), ("C", _i64), ("x_bstride", _i64),
                ("x2_bstride", _i64), ("y", _p), ("y_scale", _p), ("y_dt", ctypes.c_int), ("y_bstride", _i64),
                ("row", _i64)]


_SIGS["hca_pool_attend"] = ([_p, _p, _p, _i64, _p, _p, _p, ctypes.c_int, _i32, _p, _p, _p, _i64, _i32, _p, _i64, _i64,
                             _i32, _i32, _i64, _i64, _i64, _i64, ctypes.c_float, _p, _p, _p,
                             ctypes.POINTER(ctypes.c_size_t), _p], ctypes.c_int)
_SIGS["csa_pool_index_topk"] = ([ctypes.POINTER(BlockPool), _p, ctypes.c_int, _p, _p, _p, ctypes.c_int, _p, _i64,
                                 _i64, _i32, _i32, _i64, _i64, _i32, _i32, _p, _p, _p,
                                 ctypes.POINTER(ctypes.c_size_t), _p], ctypes.c_int)


class LibError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def load_library(path: str) -> ctypes.CDLL:
    """Load a build of the C library and declare its entry points."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m long_context_attention_25_amd.build`")
    cdll = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(cdll, name)
        fn.argtypes = args
        fn.restype = res
    return cdll


def lib() -> ctypes.CDLL:
    """The loaded C library (torch is imported first so that one HIP runtime is shared)."""
    global _lib
    if _lib is None:
        _lib = load_library(LIB_PATH)
    return _lib


class use_library:
    """Route the binding's calls through another build (e.g. DEBUG_LIB_PATH) inside a with block."""

    def __init__(self, path: str):
        self.cdll = load_library(path)

    def __enter__(self):
        global _lib
        self.saved = lib()
        _lib = self.cdll
        return self.cdll

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def debug_flags() -> int:
    """Kernel-side check bits recorded since the last read (debug build loaded; see use_library)."""
    v = ctypes.c_uint32(0)
    _check(lib().dsv4_debug_flags(ctypes.byref(v)))
    return v.value


def _check(status: int) -> None:
    if status != 0:
        raise LibError(status, lib().dsv4_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _contig(**tensors) -> None:
    """The kernels read these tensors as packed row-major arrays."""
    for name, t in tensors.items():
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _dt(t) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float8_e4m3fn:
        return FP8_E4M3
    if t.dtype == torch.uint8:
        return MXFP4
    raise TypeError(f"unsupported dtype {t.dtype}")


def _workspace(query, workspace):
    """Run the size query; return (device buffer or None, size argument for the real call)."""
    n = ctypes.c_size_t(0)
    _check(query(n))
    if n.value == 0:
        return None, None
    if workspace is None or workspace.numel() < n.value:
        workspace = torch.empty(n.value, dtype=torch.uint8, device="cuda")
    n.value = workspace.numel()
    return workspace, ctypes.byref(n)


def csa_compress(x, gate, pos_bias, m: int, y_dtype=torch.bfloat16, out=None, out_scale=None):
    """Softmax-gated pooling of disjoint blocks of m tokens: x [B,T,C] -> y [B,T/m,C].

    y_dtype: torch.float32 / torch.bfloat16 / torch.float8_e4m3fn, or MXFP4_DTYPE (returns
    (codes [B,T/m,C/2] uint8, scales [B,T/m,C/32] uint8)), or FP8_KV_DTYPE (x = K|V side by
    side; returns FP8 K|V rows [B,T/m,C+64] uint8; out_scale: optional 2 device bytes, the
    E8M0 exponents of the K and V codes).  `out` may be a [B, rows, ...] view with rows >= T/m
    (e.g. the tail of a cache); its batch stride is passed through.
    """
    if not (gate.is_contiguous() and pos_bias.is_contiguous()):
        raise ValueError("gate [B, T] and pos_bias [m] must be contiguous")
    B, T, C = x.shape
    nb = T // m
    if y_dtype == MXFP4_DTYPE:
        ydt = MXFP4
        if out is None:
            out = torch.empty((B, nb, C // 2), dtype=torch.uint8, device=x.device)
            out_scale = torch.empty((B, nb, C // 32), dtype=torch.uint8, device=x.device)
    elif y_dtype == FP8_KV_DTYPE:
        ydt = FP8_KV
        if out is None:
            out = torch.empty((B, nb, C + FP8_ROPE_DIMS), dtype=torch.uint8, device=x.device)
        if out.dtype != torch.uint8 or out.stride(-1) != 1 or (out.dim() == 3 and out.stride(1) != C + FP8_ROPE_DIMS):
            raise ValueError("FP8 K|V rows: out must be uint8 with contiguous rows of C + 64 bytes")
    else:
        ydt = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3}[y_dtype]
        if out is None:
            out = torch.empty((B, nb, C), dtype=y_dtype, device=x.device)
    y_bs = out.stride(0) // out.stride(1) if out.dim() == 3 and B > 0 else 0
    x_bs = x.stride(0) // x.stride(1) if B > 0 else 0
    _check(lib().csa_compress(_ptr(x), _dt(x), _ptr(gate), _ptr(pos_bias), B, T, C, m, x_bs, _ptr(out),
                              _ptr(out_scale), ydt, y_bs, _stream()))
    return (out, out_scale) if ydt == MXFP4 else out


def csa_compress2(x, x2, gate, pos_bias, m: int, out, out2, out2_scale, out_scale=None, fp8_kv=False):
    """Pool x [B,T,C] (bf16) into `out` (bf16 [B,rows,C], or FP8 K|V rows [B,rows,C+64] uint8
    with fp8_kv=True and optional 2-byte `out_scale`) and x2 [B,T,C2] (bf16) into MXFP4
    `out2` [B,rows,C2/2] + `out2_scale` [B,rows,C2/32], with the same gate [B,T] and pos_bias
    [m], in one launch.  Outputs may be [B, rows, ...] views (e.g. a cache's tail)."""
    if not (gate.is_contiguous() and pos_bias.is_contiguous()):
        raise ValueError("gate [B, T] and pos_bias [m] must be contiguous")
    B, T, C = x.shape
    C2 = x2.shape[2]
    if x2.shape[:2] != (B, T) or x.dtype != torch.bfloat16 or x2.dtype != torch.bfloat16:
        raise ValueError("x and x2 must be bf16 [B, T, .] over the same tokens")
    bs = lambda t: t.stride(0) // t.stride(1) if B > 0 else 0
    ydt = FP8_KV if fp8_kv else _dt(out)
    _check(lib().csa_compress2(_ptr(x), _ptr(x2), BF16, _ptr(gate), _ptr(pos_bias), B, T, m, C, bs(x), _ptr(out),
                               _ptr(out_scale), ydt, bs(out), C2, bs(x2), _ptr(out2), _ptr(out2_scale), MXFP4,
                               bs(out2), _stream()))
    return out, (out2, out2_scale)


def kv_cache_append(x_new, gate_new, pos, win, win_gate, pos_bias, m: int, cache, cache_scale=None,
                    cache_dtype=None):
    """One decode step of cache maintenance: x_new [B,C] (gate_new [B] f32, pos [B] int32)
    goes to row pos % L of the ring window win [B,L,C] / win_gate [B,L], and a block that
    the new token completes is pooled into its row of `cache` ([B,N,C] of f32/bf16/e4m3, or
    MXFP4 codes [B,N,C/2] uint8 with cache_scale [B,N,C/32], or with cache_dtype=FP8_KV_DTYPE
    FP8 K|V rows [B,N,C+64] uint8 with optional cache_scale = 2 E8M0 bytes).  Attend over such
    a window with win_pos0=None.
    """
    for t in (x_new, gate_new, pos, win, win_gate, pos_bias):
        if not t.is_contiguous():
            raise ValueError("x_new, gate_new, pos, win, win_gate and pos_bias must be contiguous")
    B, L, C = win.shape
    if x_new.shape != (B, C) or x_new.dtype != win.dtype:
        raise ValueError("x_new must be [B, C] with the window's dtype")
    if cache.stride(-1) != 1 or (cache.dim() == 3 and cache.stride(1) != cache.shape[2]):
        raise ValueError("cache rows must be contiguous")
    if cache_dtype == FP8_KV_DTYPE:
        ydt = FP8_KV
    else:
        ydt = MXFP4 if cache_scale is not None else _dt(cache)
    N = cache.shape[1]
    y_bs = cache.stride(0) // cache.stride(1) if B > 0 else 0
    _check(lib().kv_cache_append(_ptr(x_new), _dt(x_new), _ptr(gate_new), _ptr(pos), B, C, _ptr(win), _ptr(win_gate),
                                 L, _ptr(pos_bias), m, _ptr(cache), _ptr(cache_scale), ydt, N, y_bs, _stream()))


def _index_args(qi, wi, ki, q_pos, m, k, ki_scale, N, with_scores, out_idx, out_score, qi_scale):
    """Checked arguments of csa_index_topk (and of csa_pool_index_topk after its pool)."""
    B, Q, HI, DI = qi.shape
    if qi.dtype == torch.uint8:
        DI *= 2
        if (qi_scale is None or not qi.is_contiguous() or not qi_scale.is_contiguous()
                or qi_scale.data_ptr() != qi.data_ptr() + qi.numel()):
            raise ValueError("MXFP4 queries: qi_scale must follow the codes qi in the same allocation")
    _contig(qi=qi, wi=wi, q_pos=q_pos, qi_scale=qi_scale, out_idx=out_idx, out_score=out_score)
    packed = {torch.float32: DI, torch.bfloat16: DI, torch.float8_e4m3fn: DI, torch.uint8: DI // 2}.get(ki.dtype)
    if ki.dim() != 3 or ki.stride(2) != 1 or ki.stride(1) != packed:
        raise ValueError("ki rows must be packed: [B, rows, DI] (MXFP4: [B, rows, DI/2] bytes) with unit strides "
                         "inside a row")
    if ki_scale is not None and (ki_scale.stride(2) != 1 or ki_scale.stride(1) != DI // 32
                                 or ki_scale.stride(0) // ki_scale.stride(1) != ki.stride(0) // ki.stride(1)):
        raise ValueError("ki_scale rows must be packed [B, rows, DI/32] with the batch stride of ki")
    rows = ki.shape[1]
    N = rows if N is None else N
    kdt = _dt(ki)
    k_bs = ki.stride(0) // ki.stride(1) if B > 0 else 0
    if out_idx is None:
        out_idx = torch.empty((B, Q, k), dtype=torch.int32, device=qi.device)
    if with_scores and out_score is None:
        out_score = torch.empty((B, Q, k), dtype=torch.float32, device=qi.device)
    args = (_ptr(qi), _dt(qi), _ptr(wi), _ptr(ki), _ptr(ki_scale), kdt, _ptr(q_pos), B, Q, HI, DI, N, k_bs, m, k,
            _ptr(out_idx), _ptr(out_score))
    return args, out_idx, out_score


def csa_index_topk(qi, wi, ki, q_pos, m: int, k: int, ki_scale=None, N=None, with_scores=False, workspace=None,
                   out_idx=None, out_score=None, qi_scale=None):
    """Indexer scores + per-query top-k.  qi [B,Q,HI,DI], wi [B,Q,HI] f32, ki [B,rows,DI]
    (or MXFP4 codes [B,rows,DI/2] uint8 with ki_scale [B,rows,DI/32]), q_pos [B,Q] int32.
    MXFP4 queries: qi codes [B,Q,HI,DI/2] uint8 and qi_scale [B,Q,HI,DI/32], stored right
    after the codes in one allocation.
    Returns idx [B,Q,k] int32 (and scores [B,Q,k] f32 with with_scores)."""
    args, out_idx, out_score = _index_args(qi, wi, ki, q_pos, m, k, ki_scale, N, with_scores, out_idx, out_score,
                                           qi_scale)
    ws, n = _workspace(lambda n: lib().csa_index_topk(*args, None, ctypes.byref(n), _stream()), workspace)
    _check(lib().csa_index_topk(*args, _ptr(ws), n, _stream()))
    return (out_idx, out_score) if with_scores else out_idx


def csa_pool_index_topk(x, x2, gate, pos_bias, row: int, kv_cache, qi, wi, ki, q_pos, m: int, k: int, ki_scale,
                        kv_cache_scale=None, fp8_kv=False, N=None, with_scores=False, workspace=None, out_idx=None,
                        out_score=None, qi_scale=None):
    """csa_compress2 of each sequence's newest block followed by csa_index_topk, in one launch:
    x [B,m,C] raw K|V rows and x2 [B,m,DI] raw indexer-key rows (bf16, views of larger
    buffers allowed), gate [B,m], pos_bias [m]; the pooled entry goes to row `row` of
    kv_cache ([B,rows,C] bf16, or FP8 K|V rows [B,rows,C+64] uint8 with fp8_kv=True and
    kv_cache_scale) and of the MXFP4 key cache ki / ki_scale, which is then scored as by
    csa_index_topk (same arguments and results)."""
    if not (gate.is_contiguous() and pos_bias.is_contiguous()):
        raise ValueError("gate [B, m] and pos_bias [m] must be contiguous")
    B, T, C = x.shape
    if T != m or x2.shape[:2] != (B, m) or x.dtype != torch.bfloat16 or x2.dtype != torch.bfloat16:
        raise ValueError("x and x2 must be bf16 [B, m, .]: the newest block of each sequence")
    if x.stride(2) != 1 or x.stride(1) != C or x2.stride(2) != 1 or x2.stride(1) != x2.shape[2]:
        raise ValueError("x and x2 rows must be packed")
    if kv_cache.dim() != 3 or kv_cache.stride(2) != 1 or kv_cache.stride(1) != kv_cache.shape[2]:
        raise ValueError("kv_cache rows must be packed")
    args, out_idx, out_score = _index_args(qi, wi, ki, q_pos, m, k, ki_scale, N, with_scores, out_idx, out_score,
                                           qi_scale)
    bs = lambda t: t.stride(0) // t.stride(1) if B > 0 else 0
    pool = BlockPool(_ptr(x), _ptr(x2), _ptr(gate), _ptr(pos_bias), C, bs(x), bs(x2),
                     ctypes.c_void_p(kv_cache[:, row].data_ptr()) if B > 0 else None, _ptr(kv_cache_scale),
                     FP8_KV if fp8_kv else _dt(kv_cache), bs(kv_cache), row)
    ws, n = _workspace(lambda n: lib().csa_pool_index_topk(ctypes.byref(pool), *args, None, ctypes.byref(n),
                                                           _stream()), workspace)
    _check(lib().csa_pool_index_topk(ctypes.byref(pool), *args, _ptr(ws), n, _stream()))
    return (out_idx, out_score) if with_scores else out_idx


def _attend_common(q, kc, vc, kw, vw, win_pos0, q_pos, N):
    """Sizes and strides of the key/value tensors: rows may be wider than D (e.g. K and V
    side by side in one [.., 2D] buffer), the last dimension must be contiguous."""
    B, Q, H, D = q.shape
    N = kc.shape[1] if N is None else N
    _contig(q=q, q_pos=q_pos, win_pos0=win_pos0)
    if kc.stride(-1) != 1 or kw.stride(-1) != 1 or kc.stride() != vc.stride() or kw.stride() != vw.stride():
        raise ValueError("kc/vc and kw/vw must share strides and have a contiguous last dimension")
    kv_rs, w_rs = kc.stride(1), kw.stride(1)
    kv_bs = kc.stride(0) // kv_rs if B > 0 else 0
    L = kw.shape[1]
    if B > 1 and kw.stride(0) != L * w_rs:
        raise ValueError("kw/vw batches must be L rows apart")
    return B, Q, H, D, N, kv_bs, L, kv_rs, w_rs


def csa_attend(q, kc, vc, idx, kw, vw, win_pos0, W: int, q_pos, scale: float, N=None, workspace=None, out=None,
               lse=None):
    """One softmax over the listed compressed entries and the window rows (win_pos0=None:
    a ring window, position p in row p % L).  Returns (o [B,Q,H,D] in q's dtype, lse [B,Q,H] f32)."""
    B, Q, H, D, N, kv_bs, L, kv_rs, w_rs = _attend_common(q, kc, vc, kw, vw, win_pos0, q_pos, N)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device) if lse is None else lse
    _contig(idx=idx, out=out, lse=lse)
    args = (_ptr(q), _ptr(kc), _ptr(vc), _dt(q), _ptr(idx), idx.shape[2], _ptr(kw), _ptr(vw), _ptr(win_pos0), L, W,
            _ptr(q_pos), B, Q, H, D, N, kv_bs, kv_rs, w_rs, float(scale), _ptr(out), _ptr(lse))
    ws, n = _workspace(lambda n: lib().csa_attend(*args, None, ctypes.byref(n), _stream()), workspace)
    _check(lib().csa_attend(*args, _ptr(ws), n, _stream()))
    return out, lse


def hca_attend(q, kc, vc, m: int, kw, vw, win_pos0, W: int, q_pos, scale: float, N=None, workspace=None, out=None,
               lse=None):
    """One softmax over every visible compressed entry and the window rows."""
    B, Q, H, D, N, kv_bs, L, kv_rs, w_rs = _attend_common(q, kc, vc, kw, vw, win_pos0, q_pos, N)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device) if lse is None else lse
    _contig(out=out, lse=lse)
    args = (_ptr(q), _ptr(kc), _ptr(vc), _dt(q), m, _ptr(kw), _ptr(vw), _ptr(win_pos0), L, W, _ptr(q_pos), B, Q, H,
            D, N, kv_bs, kv_rs, w_rs, float(scale), _ptr(out), _ptr(lse))
    ws, n = _workspace(lambda n: lib().hca_attend(*args, None, ctypes.byref(n), _stream()), workspace)
    _check(lib().hca_attend(*args, _ptr(ws), n, _stream()))
    return out, lse


def hca_pool_attend(x, gate, pos_bias, q, kc, vc, m: int, kw, vw, win_pos0, W: int, q_pos, scale: float, N=None,
                    workspace=None, out=None, lse=None):
    """csa_compress of each sequence's newest block followed by hca_attend, in one launch:
    x [B,m,2D] raw K|V rows (bf16, a view of a larger buffer allowed), gate [B,m], pos_bias
    [m]; the pooled entry goes to row N-1 of the cache whose K and V halves are kc and vc
    (views of one [B,rows,2D] buffer), then every visible entry and the window are attended."""
    if not (gate.is_contiguous() and pos_bias.is_contiguous()):
        raise ValueError("gate [B, m] and pos_bias [m] must be contiguous")
    B, T, C2 = x.shape
    if T != m or x.dtype != torch.bfloat16 or x.stride(2) != 1 or x.stride(1) != C2:
        raise ValueError("x must be packed bf16 rows [B, m, 2D]: the newest block of each sequence")
    B_, Q, H, D, N, kv_bs, L, kv_rs, w_rs = _attend_common(q, kc, vc, kw, vw, win_pos0, q_pos, N)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B_, Q, H), dtype=torch.float32, device=q.device) if lse is None else lse
    _contig(out=out, lse=lse)
    args = (_ptr(x), _ptr(gate), _ptr(pos_bias), x.stride(0) // x.stride(1) if B > 0 else 0, _ptr(q), _ptr(kc),
            _ptr(vc), _dt(q), m, _ptr(kw), _ptr(vw), _ptr(win_pos0), L, W, _ptr(q_pos), B_, Q, H, D, N, kv_bs, kv_rs,
            w_rs, float(scale), _ptr(out), _ptr(lse))
    ws, n = _workspace(lambda n: lib().hca_pool_attend(*args, None, ctypes.byref(n), _stream()), workspace)
    _check(lib().hca_pool_attend(*args, _ptr(ws), n, _stream()))
    return out, lse


def _fp8kv_common(q, kc, vc, kw, vw, N, d_rope):
    """Byte strides of FP8 K/V rows (uint8 tensors [B, rows, bytes], last dimension
    contiguous): K rows of D + d_rope bytes, V rows of D bytes, either each in its own
    tensor (natural strides) or sharing one row stride (e.g. K and V side by side)."""
    B, Q, H, D = q.shape
    N = kc.shape[1] if N is None else N
    _contig(q=q)
    for t in (kc, vc, kw, vw):
        if t.dtype != torch.uint8 or t.stride(-1) != 1:
            raise ValueError("FP8 K/V rows are uint8 tensors with a contiguous last dimension")
    if kc.shape[-1] != D + d_rope or vc.shape[-1] != D or kw.shape[-1] != D + d_rope or vw.shape[-1] != D:
        raise ValueError("K rows must hold D + d_rope bytes and V rows D bytes")

    def rows(k, v):
        if k.stride(1) == v.stride(1):
            rs = k.stride(1)
            if B > 1 and k.stride(0) != v.stride(0):
                raise ValueError("K and V batches must be equally far apart")
            return rs, (k.stride(0) // rs if B > 0 else 0)
        if k.stride(1) != D + d_rope or v.stride(1) != D:
            raise ValueError("K and V rows must share a row stride or be packed")
        kb, vb = k.stride(0) // k.stride(1), v.stride(0) // v.stride(1)
        if B > 1 and kb != vb:
            raise ValueError("K and V batches must hold the same number of rows")
        return 0, (kb if B > 0 else 0)

    kv_rs, kv_bs = rows(kc, vc)
    w_rs, w_bs = rows(kw, vw)
    L = kw.shape[1]
    if B > 1 and w_bs != L:
        raise ValueError("kw/vw batches must be L rows apart")
    return B, Q, H, D, N, kv_bs, L, kv_rs, w_rs


def csa_attend_fp8kv(q, kc, vc, idx, kw, vw, win_pos0, W: int, q_pos, scale: float, k_scale: float = 1.0,
                     v_scale: float = 1.0, d_rope: int = FP8_ROPE_DIMS, N=None, workspace=None, out=None, lse=None):
    """csa_attend over FP8 K/V rows (K: D - d_rope E4M3 codes then d_rope bf16 values; V: D
    E4M3 codes; decoded K codes x k_scale, V codes x v_scale).  q and the output are bf16."""
    B, Q, H, D, N, kv_bs, L, kv_rs, w_rs = _fp8kv_common(q, kc, vc, kw, vw, N, d_rope)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device) if lse is None else lse
    _contig(idx=idx, q_pos=q_pos, win_pos0=win_pos0, out=out, lse=lse)
    args = (_ptr(q), _ptr(kc), _ptr(vc), _ptr(idx), idx.shape[2], _ptr(kw), _ptr(vw), _ptr(win_pos0), L, W,
            _ptr(q_pos), B, Q, H, D, d_rope, N, kv_bs, kv_rs, w_rs, float(k_scale), float(v_scale), float(scale),
            _ptr(out), _ptr(lse))
    ws, n = _workspace(lambda n: lib().csa_attend_fp8kv(*args, None, ctypes.byref(n), _stream()), workspace)
    _check(lib().csa_attend_fp8kv(*args, _ptr(ws), n, _stream()))
    return out, lse


def hca_attend_fp8kv(q, kc, vc, m: int, kw, vw, win_pos0, W: int, q_pos, scale: float, k_scale: float = 1.0,
                     v_scale: float = 1.0, d_rope: int = FP8_ROPE_DIMS, N=None, workspace=None, out=None, lse=None):
    """hca_attend over FP8 K/V rows (layout as csa_attend_fp8kv)."""
    B, Q, H, D, N, kv_bs, L, kv_rs, w_rs = _fp8kv_common(q, kc, vc, kw, vw, N, d_rope)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device) if lse is None else lse
    _contig(q_pos=q_pos, win_pos0=win_pos0, out=out, lse=lse)
    args = (_ptr(q), _ptr(kc), _ptr(vc), m, _ptr(kw), _ptr(vw), _ptr(win_pos0), L, W, _ptr(q_pos), B, Q, H, D,
            d_rope, N, kv_bs, kv_rs, w_rs, float(k_scale), float(v_scale), float(scale), _ptr(out), _ptr(lse))
    ws, n = _workspace(lambda n: lib().hca_attend_fp8kv(*args, None, ctypes.byref(n), _stream()), workspace)
    _check(lib().hca_attend_fp8kv(*args, _ptr(ws), n, _stream()))
    return out, lse


def lse_merge(o_parts, lse_parts, out_dtype=torch.float32, out=None, lse_out=None):
    """Merge partial attentions over disjoint key sets: o_parts [P,R,D] f32, lse_parts [P,R] f32."""
    P, R, D = o_parts.shape
    out = torch.empty((R, D), dtype=out_dtype, device=o_parts.device) if out is None else out
    lse_out = torch.empty((R,), dtype=torch.float32, device=o_parts.device) if lse_out is None else lse_out
    _contig(o_parts=o_parts, lse_parts=lse_parts, out=out, lse_out=lse_out)
    _check(lib().lse_merge(_ptr(o_parts), _ptr(lse_parts), P, R, D, _ptr(out), _dt(out), _ptr(lse_out), _stream()))
    return out, lse_out
