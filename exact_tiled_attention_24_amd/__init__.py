"""Exact tiled attention for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libfa.so`` (declared in ``include/fa.h``): it checks tensor
shapes, dtypes and devices, allocates outputs through torch, and passes raw device pointers
and the current HIP stream to the C ABI. Every step of the computation runs in the HIP
kernels; there is no fallback. If the library is missing or fails to load, every call
raises.

Entry points (same names as the C ABI):
    fa_fwd(q, k, v, scale=None, causal=False, out=None, return_stats=False)
    fa_decode_splitk(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, ...)
    fa_decode_splitk_noalloc(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, out, ...)
    fa_fwd_paged(q, k_cache, v_cache, block_table, seq_lens, scale=None, causal=True, ...)
    fa_fwd_block_sparse(q, k, v, block_offsets, block_indices, scale=None, causal=False, ...)
    fa_bwd(q, k, v, o, dout, m, l, scale=None, causal=False, workspace=None)
    fa_fwd_fp8(q_e4m3, k_e4m3, v_bf16_or_e4m3, scale=None, causal=False, out=None, return_stats=False)
    fa_merge(o_parts, m_parts, l_parts, out_dtype=torch.float32, return_stats=False)
    fa_decode_workspace_bytes(...), fa_decode_plan_splits(...), fa_status_string(code)
"""

from __future__ import annotations

import ctypes
import math
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARGUMENT = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_WORKSPACE_TOO_SMALL = 3
FA_ERR_HIP = 4
FA_F32 = 0
FA_BF16 = 1
FA_E4M3 = 2

_lib = None


class FaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {fa_status_string(code)}")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so and declare its C signatures. Raises if it is not built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m exact_tiled_attention_24_amd.build` "
            "(the HIP library is required, there is no fallback)")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.fa_fwd.restype = i32
    lib.fa_decode_splitk.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                     i32, i32, f32, i32, vp, sz, vp]
    lib.fa_decode_splitk.restype = i32
    lib.fa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_decode_splitk_noalloc.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                             i32, i32, i32, f32, i32, vp]
    lib.fa_decode_splitk_noalloc.restype = i32
    lib.fa_decode_noalloc_max_bytes.argtypes = []
    lib.fa_decode_noalloc_max_bytes.restype = sz
    lib.fa_decode_plan_splits.argtypes = [i32, i32, i32, i32]
    lib.fa_decode_plan_splits.restype = i32
    lib.fa_fwd_paged.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                 i32, i32, i32, i32, f32, i32, vp]
    lib.fa_fwd_paged.restype = i32
    lib.fa_fwd_block_sparse.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                        i32, i32, f32, i32, vp]
    lib.fa_fwd_block_sparse.restype = i32
    lib.fa_fwd_fp8.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.fa_fwd_fp8.restype = i32
    lib.fa_bwd.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                           f32, i32, vp, sz, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_workspace_bytes.argtypes = [i32, i32, i32]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_merge.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, vp]
    lib.fa_merge.restype = i32
    lib.fa_status_string.argtypes = [i32]
    lib.fa_status_string.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def fa_status_string(code: int) -> str:
    return load_library().fa_status_string(int(code)).decode()


def _check(code: int, where: str) -> None:
    if code != FA_OK:
        raise FaError(code, where)


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    dev = ts[0].device
    for t in ts:
        if t is not None and t.device != dev:
            raise ValueError("all tensors must be on the same device")


def fa_fwd(q, k, v, scale=None, causal=False, out=None, return_stats=False):
    """Tiled attention forward. q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (bf16 or f32).

    Returns O [B, Hq, N, d] in q's dtype, or (O, m, l) with float32 [B, Hq, N] statistics in
    natural-log units when ``return_stats``.
    """
    torch = _torch()
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    Hkv = k.shape[1]
    o = torch.empty_like(q) if out is None else out
    m = l = None
    if return_stats:
        m = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
        l = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _require_gpu(q, k, v, o, m, l)
    if o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        code = lib.fa_fwd(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(m), _ptr(l),
                          B, Hq, Hkv, N, d, scale, 1 if causal else 0, _stream(q.device))
    _check(code, "fa_fwd")
    return (o, m, l) if return_stats else o


def fa_decode_workspace_bytes(B, Hq, d, page_size, max_seq_len, num_splits=0) -> int:
    return int(load_library().fa_decode_workspace_bytes(B, Hq, d, page_size, max_seq_len,
                                                         num_splits))


def fa_decode_plan_splits(B, Hkv, page_size, max_seq_len) -> int:
    return int(load_library().fa_decode_plan_splits(B, Hkv, page_size, max_seq_len))


def fa_decode_splitk(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, scale=None,
                     num_splits=0, out=None, workspace=None):
    """Single-query decode over a paged KV cache, split across the KV sequence.

    q: [B, Hq, d] bf16; k_cache, v_cache: [num_pages, Hkv, page_size, d] bf16;
    block_table: int32 [B, max_pages_per_seq]; seq_lens: int32 [B] (both on the GPU).
    Returns O [B, Hq, d] bf16. ``workspace`` (uint8, on the GPU) is allocated if omitted.
    """
    torch = _torch()
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B, Hq, d]; caches [num_pages, Hkv, page_size, d]")
    B, Hq, d = q.shape
    num_pages, Hkv, page_size, dk = k_cache.shape
    if dk != d:
        raise ValueError("head dimension mismatch between q and the cache")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages_per_seq] and seq_lens [B]")
    o = torch.empty_like(q) if out is None else out
    need = fa_decode_workspace_bytes(B, Hq, d, page_size, int(max_seq_len), int(num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _require_gpu(q, k_cache, v_cache, block_table, seq_lens, o, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        code = lib.fa_decode_splitk(
            _dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seq_lens), _ptr(o), B, Hq, Hkv, d, page_size, num_pages, block_table.shape[1],
            int(max_seq_len), scale, int(num_splits), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(code, "fa_decode_splitk")
    return o


def fa_decode_noalloc_max_bytes() -> int:
    return int(load_library().fa_decode_noalloc_max_bytes())


def fa_decode_splitk_noalloc(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, out,
                             scale=None, num_splits=0):
    """fa_decode_splitk without a workspace: the library's static per-device scratch holds the
    partials, and nothing is allocated (``out``, bf16 [B, Hq, d], is the caller's). Calls that
    overlap in time on one device race on that scratch: keep them on one stream."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B, Hq, d]; caches [num_pages, Hkv, page_size, d]")
    B, Hq, d = q.shape
    num_pages, Hkv, page_size, dk = k_cache.shape
    if dk != d:
        raise ValueError("head dimension mismatch between q and the cache")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages_per_seq] and seq_lens [B]")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    _require_gpu(q, k_cache, v_cache, block_table, seq_lens, out)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        code = lib.fa_decode_splitk_noalloc(
            _dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seq_lens), _ptr(out), B, Hq, Hkv, d, page_size, num_pages, block_table.shape[1],
            int(max_seq_len), scale, int(num_splits), _stream(q.device))
    _check(code, "fa_decode_splitk_noalloc")
    return out


def fa_fwd_paged(q, k_cache, v_cache, block_table, seq_lens, scale=None, causal=True, out=None,
                 return_stats=False, q_lens=None):
    """Chunked prefill over a paged KV cache: each sequence's newest Nq tokens attend to its
    whole cache (query i at position seq_lens[b] - Nq + i).

    q: [B, Hq, Nq, d] bf16; k_cache, v_cache: [num_pages, Hkv, 16, d] bf16; block_table:
    int32 [B, max_pages_per_seq]; seq_lens: int32 [B] (all on the GPU). Returns O [B, Hq, Nq,
    d] bf16, or (O, m, l) with float32 [B, Hq, Nq] statistics when ``return_stats``.
    ``q_lens`` (int32 [B] on the GPU): new tokens per sequence, in the first rows of q; the
    other rows of the outputs are not written.
    """
    torch = _torch()
    lib = load_library()
    if q.dim() != 4 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [B, Hq, Nq, d]; caches [num_pages, Hkv, page_size, d]")
    B, Hq, Nq, d = q.shape
    num_pages, Hkv, page_size, dk = k_cache.shape
    if dk != d:
        raise ValueError("head dimension mismatch between q and the cache")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B or seq_lens.shape != (B,):
        raise ValueError("block_table must be [B, max_pages_per_seq] and seq_lens [B]")
    o = torch.empty_like(q) if out is None else out
    m = l = None
    if return_stats:
        m = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
        l = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if q_lens is not None and (q_lens.dtype != torch.int32 or q_lens.shape != (B,)):
        raise ValueError("q_lens must be int32 [B]")
    _require_gpu(q, k_cache, v_cache, block_table, seq_lens, o, m, l, q_lens)
    if o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        code = lib.fa_fwd_paged(
            _dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(seq_lens), _ptr(q_lens), _ptr(o), _ptr(m), _ptr(l), B, Hq, Hkv, Nq, d, page_size, num_pages,
            block_table.shape[1], scale, 1 if causal else 0, _stream(q.device))
    _check(code, "fa_fwd_paged")
    return (o, m, l) if return_stats else o


def fa_fwd_fp8(q, k, v, scale=None, causal=False, out=None, return_stats=False):
    """Forward with fp8 queries and keys. q: uint8 e4m3 codes [B, Hq, N, d]; k: uint8 e4m3 codes
    [B, Hkv, N, d]; v: [B, Hkv, N, d] bf16, or uint8 e4m3 codes (then P is rounded to e4m3 and
    P V runs on the fp8 matrix cores too). Returns O bf16 [B, Hq, N, d] (or (O, m, l))."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    if q.dtype != torch.uint8 or k.dtype != torch.uint8:
        raise TypeError("q and k must be uint8 e4m3 codes")
    if v.dtype == torch.bfloat16:
        v_dt = FA_BF16
    elif v.dtype == torch.uint8:
        v_dt = FA_E4M3
    else:
        raise TypeError("v must be bfloat16 or uint8 e4m3 codes")
    B, Hq, N, d = q.shape
    if k.shape[0] != B or k.shape[2:] != q.shape[2:]:
        raise ValueError("shape mismatch")
    o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=q.device) if out is None else out
    m = l = None
    if return_stats:
        m = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
        l = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _require_gpu(q, k, v, o, m, l)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        code = lib.fa_fwd_fp8(v_dt, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(m), _ptr(l), B, Hq,
                              k.shape[1], N, d, scale, 1 if causal else 0, _stream(q.device))
    _check(code, "fa_fwd_fp8")
    return (o, m, l) if return_stats else o


def fa_bwd_workspace_bytes(B, Hq, N) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, Hq, N))


def fa_bwd(q, k, v, o, dout, m, l, scale=None, causal=False, workspace=None):
    """Backward of fa_fwd: returns (dq, dk, dv) in q's dtype (bf16). q, o, dout: [B, Hq, N, d];
    k, v: [B, Hkv, N, d]; m, l: the float32 [B, Hq, N] statistics fa_fwd returned."""
    torch = _torch()
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    B, Hq, N, d = q.shape
    if o.shape != q.shape or dout.shape != q.shape or k.shape[0] != B or k.shape[2:] != q.shape[2:]:
        raise ValueError("shape mismatch")
    if m.shape != (B, Hq, N) or l.shape != (B, Hq, N) or m.dtype != torch.float32 or l.dtype != torch.float32:
        raise ValueError("m and l must be float32 [B, Hq, N]")
    if q.dtype != torch.bfloat16:
        raise TypeError(f"fa_bwd takes bfloat16 tensors, got q of dtype {q.dtype}")
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}; fa_bwd needs every tensor in q's dtype "
                            f"({q.dtype})")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if workspace is None:
        workspace = torch.empty(max(fa_bwd_workspace_bytes(B, Hq, N), 16), dtype=torch.uint8,
                                device=q.device)
    _require_gpu(q, k, v, o, dout, m, l, dq, dk, dv, workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        code = lib.fa_bwd(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(m),
                          _ptr(l), _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, k.shape[1], N, d, scale,
                          1 if causal else 0, _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(code, "fa_bwd")
    return dq, dk, dv


SPARSE_BLOCK_Q = 256
SPARSE_BLOCK_K = 64


def fa_fwd_block_sparse(q, k, v, block_offsets, block_indices, scale=None, causal=False,
                        out=None, return_stats=False):
    """Block-sparse forward: query block qb (256 rows) of head (b, h) attends only to the
    64-key blocks block_indices[block_offsets[r]:block_offsets[r + 1]],
    r = (b * Hq + h) * ceil(N / 256) + qb. q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (bf16);
    block_offsets, block_indices: int32 on the GPU. Returns O, or (O, m, l) with
    ``return_stats``.
    """
    torch = _torch()
    lib = load_library()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if block_offsets.dtype != torch.int32 or block_indices.dtype != torch.int32:
        raise TypeError("block_offsets and block_indices must be int32")
    nqb = -(-N // SPARSE_BLOCK_Q)
    if block_offsets.dim() != 1 or block_offsets.numel() != B * Hq * nqb + 1:
        raise ValueError("block_offsets must hold B * Hq * ceil(N / 256) + 1 entries")
    Hkv = k.shape[1]
    o = torch.empty_like(q) if out is None else out
    m = l = None
    if return_stats:
        m = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
        l = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _require_gpu(q, k, v, o, block_offsets, block_indices, m, l)
    if o.shape != q.shape or o.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):
        code = lib.fa_fwd_block_sparse(
            _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(m), _ptr(l),
            _ptr(block_offsets), _ptr(block_indices), block_indices.numel(), B, Hq, Hkv, N, d,
            scale, 1 if causal else 0, _stream(q.device))
    _check(code, "fa_fwd_block_sparse")
    return (o, m, l) if return_stats else o


def fa_merge(o_parts, m_parts, l_parts, out_dtype=None, return_stats=False, out=None):
    """Merge S partials: o_parts float32 [S, R, d], m_parts / l_parts float32 [S, R]."""
    torch = _torch()
    lib = load_library()
    if o_parts.dim() != 3 or m_parts.shape != o_parts.shape[:2] or l_parts.shape != m_parts.shape:
        raise ValueError("o_parts must be [S, R, d] and m_parts, l_parts [S, R]")
    for t in (o_parts, m_parts, l_parts):
        if t.dtype != torch.float32:
            raise TypeError("partials must be float32")
    S, R, d = o_parts.shape
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    o = torch.empty((R, d), dtype=out_dtype, device=o_parts.device) if out is None else out
    m = l = None
    if return_stats:
        m = torch.empty((R,), dtype=torch.float32, device=o_parts.device)
        l = torch.empty((R,), dtype=torch.float32, device=o_parts.device)
    _require_gpu(o_parts, m_parts, l_parts, o, m, l)
    with torch.cuda.device(o_parts.device):
        code = lib.fa_merge(_dtype_code(o), _ptr(o_parts), _ptr(m_parts), _ptr(l_parts), _ptr(o),
                            _ptr(m), _ptr(l), S, R, d, _stream(o_parts.device))
    _check(code, "fa_merge")
    return (o, m, l) if return_stats else o
