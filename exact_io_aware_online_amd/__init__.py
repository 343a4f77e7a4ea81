"""Exact IO-aware attention for MI355X (gfx950): Python binding of libfa.so.

The binding only marshals arguments: it checks dtypes, devices and
contiguity, takes raw device pointers and the current HIP stream from torch
tensors, and calls the C ABI of ``include/fa.h`` through ctypes. Every step
of the computation runs in the HIP kernels of ``libfa.so``; there is no
fallback, and calling anything here without the built library raises.
"""

import ctypes
import math
import os

__all__ = [
    "FAError",
    "lib",
    "fa_abi_version",
    "fa_status_string",
    "fa_fwd",
    "fa_fwd_window",
    "fa_fwd_varlen",
    "fa_fwd_kvcache",
    "fa_fwd_kvcache_workspace_size",
    "fa_kvcache_default_splits",
    "fa_kvcache_append_default_splits",
    "fa_fwd_kvcache_paged",
    "fa_fwd_kvcache_noalloc",
    "FA_NOALLOC_SCRATCH_BYTES",
    "fa_fwd_kvcache_append",
    "fa_fwd_kvcache_paged_append",
    "fa_fp8_padded_rows",
    "fa_quantize_fp8",
    "fa_fwd_fp8",
    "fa_bwd",
    "fa_bwd_window",
    "fa_bwd_varlen",
    "fa_bwd_workspace_size",
    "FA_DTYPE_BF16",
    "FA_DTYPE_F32",
]

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_LAUNCH = range(5)
FA_DTYPE_BF16, FA_DTYPE_F32 = 0, 1
FA_NOALLOC_SCRATCH_BYTES = 16 << 20  # the static per-GPU scratch of fa_fwd_kvcache_noalloc

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} (status {status})")


def lib():
    """The loaded libfa.so (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m exact_io_aware_online_amd.build` "
                          "(there is no fallback implementation)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.fa_abi_version.restype = i
    L.fa_abi_version.argtypes = []
    L.fa_status_string.restype = ctypes.c_char_p
    L.fa_status_string.argtypes = [i]
    L.fa_fwd.restype = i
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    L.fa_fwd_window.restype = i
    L.fa_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp]
    L.fa_fwd_varlen.restype = i
    L.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, vp]
    L.fa_fwd_kvcache.restype = i
    L.fa_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, sz, vp]
    L.fa_fwd_kvcache_noalloc.restype = i
    L.fa_fwd_kvcache_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.fa_fwd_kvcache_workspace_size.restype = sz
    L.fa_fwd_kvcache_workspace_size.argtypes = [i, i, i, i]
    L.fa_kvcache_default_splits.restype = i
    L.fa_kvcache_default_splits.argtypes = [i, i, i, i, i, i]
    L.fa_kvcache_append_default_splits.restype = i
    L.fa_kvcache_append_default_splits.argtypes = [i, i, i, i, i, i, i, i]
    L.fa_fwd_kvcache_paged.restype = i
    L.fa_fwd_kvcache_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp, sz, vp]
    L.fa_fwd_kvcache_append.restype = i
    L.fa_fwd_kvcache_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp, sz, vp]
    L.fa_fwd_kvcache_paged_append.restype = i
    L.fa_fwd_kvcache_paged_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, f,
                                              vp, sz, vp]
    L.fa_fp8_padded_rows.restype = i
    L.fa_fp8_padded_rows.argtypes = [i]
    L.fa_quantize_fp8.restype = i
    L.fa_quantize_fp8.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
    L.fa_fwd_fp8.restype = i
    L.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    L.fa_bwd_workspace_size.restype = sz
    L.fa_bwd_workspace_size.argtypes = [i, i, i]
    L.fa_bwd.restype = i
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, sz, vp]
    L.fa_bwd_window.restype = i
    L.fa_bwd_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp, sz, vp]
    L.fa_bwd_varlen.restype = i
    L.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, f, vp, sz,
                                vp]
    _lib = L
    return L


def fa_abi_version():
    return lib().fa_abi_version()


def fa_status_string(status):
    return lib().fa_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, name, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _shape(t, shape, name):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _workspace(workspace, need, device):
    """The caller's workspace (any dtype, contiguous, on `device`) or a new
    one of `need` bytes; returns (tensor or None, its size in bytes)."""
    import torch
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    if workspace is not None:
        _check(workspace, "workspace", device=device)
    return workspace, 0 if workspace is None else workspace.numel() * workspace.element_size()


def fa_fwd(q, k, v, o=None, lse=None, causal=False, scale=None, stream=None, want_lse=True):
    """Attention forward through ``fa_fwd``.

    q: (B, Nq, Hq, d); k, v: (B, Nk, Hkv, d); bf16 or float32, contiguous,
    on one GPU. ``o`` (like q) and ``lse`` ((B, Hq, Nq) float32) are
    allocated when not given. Returns (o, lse); lse is None when
    ``want_lse`` is false and no ``lse`` tensor was passed.
    """
    import torch
    if q.dtype == torch.bfloat16:
        dt = FA_DTYPE_BF16
    elif q.dtype == torch.float32:
        dt = FA_DTYPE_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be (batch, seq, heads, head_dim)")
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Nk, Hkv, d) or tuple(v.shape) != (B, Nk, Hkv, d):
        raise ValueError(f"k/v shapes {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, q.dtype, q.device)
    if o is None:
        o = torch.empty_like(q)
    _check(o, "o", q.dtype, q.device)
    if tuple(o.shape) != tuple(q.shape):
        raise ValueError("o must have q's shape")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, q.device)
        if tuple(lse.shape) != (B, Hq, Nq):
            raise ValueError("lse must be (B, Hq, Nq)")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                      int(bool(causal)), float(scale), dt, _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd")
    return o, lse


def fa_fwd_window(q, k, v, window_left=-1, window_right=-1, o=None, lse=None, scale=None, stream=None,
                  want_lse=True):
    """Bottom-right aligned local-window attention through ``fa_fwd_window``.

    q: (B, Nq, Hq, d); k, v: (B, Nk, Hkv, d); bf16. Key j is visible to
    query i iff i + (Nk - Nq) - window_left <= j <= i + (Nk - Nq) +
    window_right (negative: unlimited). Returns (o, lse (B, Hq, Nq)).
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be (batch, seq, heads, head_dim)")
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Nk, Hkv, d) or tuple(v.shape) != (B, Nk, Hkv, d):
        raise ValueError("k/v shapes do not match q")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16, q.device)
    o = torch.empty_like(q) if o is None else o
    _check(o, "o", torch.bfloat16, q.device)
    _shape(o, q.shape, "o")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, q.device)
        _shape(lse, (B, Hq, Nq), "lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                             int(window_left), int(window_right), float(scale), _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_window")
    return o, lse


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, window_left=-1, window_right=-1, o=None,
                  lse=None, scale=None, stream=None, want_lse=True):
    """Packed variable-length batch through ``fa_fwd_varlen``.

    q: (total_q, Hq, d); k, v: (total_k, Hkv, d); bf16; cu_seqlens_*:
    (B + 1,) int32 on the same GPU. Returns (o (total_q, Hq, d),
    lse (Hq, total_q)).
    """
    import torch
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be (tokens, heads, head_dim)")
    total_q, Hq, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    if tuple(v.shape) != tuple(k.shape) or k.shape[2] != d:
        raise ValueError("k/v shapes do not match q")
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, torch.bfloat16, q.device)
    for t, n in ((cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k")):
        _check(t, n, torch.int32, q.device)
    B = cu_seqlens_q.numel() - 1
    if B < 0 or cu_seqlens_q.dim() != 1 or tuple(cu_seqlens_k.shape) != (B + 1,):
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be (B + 1,)")
    o = torch.empty_like(q) if o is None else o
    _check(o, "o", torch.bfloat16, q.device)
    _shape(o, q.shape, "o")
    if lse is None and want_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, q.device)
        _shape(lse, (Hq, total_q), "lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                             B, Hq, Hkv, int(max_seqlen_q), total_q, total_k, d, int(window_left),
                             int(window_right), float(scale), _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_varlen")
    return o, lse


def fa_fwd_kvcache_workspace_size(B, Hq, d, num_splits):
    return int(lib().fa_fwd_kvcache_workspace_size(int(B), int(Hq), int(d), int(num_splits)))


def fa_kvcache_default_splits(B, Hkv, capacity, d=128, num_cus=0, wgs_per_cu=0):
    return int(lib().fa_kvcache_default_splits(int(B), int(Hkv), int(capacity), int(d), int(num_cus),
                                               int(wgs_per_cu)))


def fa_kvcache_append_default_splits(B, Nq, Hkv, Hq, capacity, d=128, num_cus=0, wgs_per_cu=0):
    return int(lib().fa_kvcache_append_default_splits(int(B), int(Nq), int(Hkv), int(Hq), int(capacity), int(d),
                                                      int(num_cus), int(wgs_per_cu)))


def fa_fwd_kvcache(q, kcache, vcache, cache_seqlens, o=None, lse=None, num_splits=None, scale=None,
                   workspace=None, stream=None, want_lse=True):
    """Split-KV decode through ``fa_fwd_kvcache``.

    q: (B, 1, Hq, d) bf16; kcache, vcache: (B, capacity, Hkv, d) bf16;
    cache_seqlens: (B,) int32 on the same GPU. ``num_splits`` defaults to
    ``fa_kvcache_default_splits``; the workspace is allocated when needed
    and not given. Returns (o (B, 1, Hq, d) bf16, lse (B, Hq) float32).
    """
    import torch
    if q.dim() != 4 or q.shape[1] != 1:
        raise ValueError("q must be (batch, 1, heads, head_dim)")
    B, _, Hq, d = q.shape
    _, cap, Hkv, dk = kcache.shape
    if dk != d or tuple(vcache.shape) != tuple(kcache.shape) or kcache.shape[0] != B:
        raise ValueError("cache shapes do not match q")
    for t, n in ((q, "q"), (kcache, "kcache"), (vcache, "vcache")):
        _check(t, n, torch.bfloat16, q.device)
    _check(cache_seqlens, "cache_seqlens", torch.int32, q.device)
    if tuple(cache_seqlens.shape) != (B,):
        raise ValueError("cache_seqlens must be (B,)")
    if num_splits is None:
        num_splits = fa_kvcache_default_splits(B, Hkv, cap, d)
    if o is None:
        o = torch.empty_like(q)
    _check(o, "o", torch.bfloat16, q.device)
    _shape(o, q.shape, "o")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, q.device)
        _shape(lse, (B, Hq), "lse")
    workspace, ws_bytes = _workspace(workspace, fa_fwd_kvcache_workspace_size(B, Hq, d, num_splits), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_kvcache(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(cache_seqlens), _ptr(o), _ptr(lse),
                              int(num_splits), B, Hq, Hkv, cap, d, float(scale), _ptr(workspace), ws_bytes,
                              _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_kvcache")
    return o, lse


def fa_fwd_kvcache_noalloc(q, kcache, vcache, cache_seqlens, o=None, lse=None, num_splits=None, scale=None,
                           stream=None, want_lse=True):
    """Split-KV decode through ``fa_fwd_kvcache_noalloc``: as
    ``fa_fwd_kvcache``, but the library keeps the split partials in its own
    static per-GPU scratch (FA_NOALLOC_SCRATCH_BYTES), so the call itself
    allocates nothing on the device. Calls that overlap on one GPU race on
    that scratch. ``o`` and ``lse`` are allocated here when not given.
    """
    import torch
    if q.dim() != 4 or q.shape[1] != 1:
        raise ValueError("q must be (batch, 1, heads, head_dim)")
    B, _, Hq, d = q.shape
    if kcache.dim() != 4:
        raise ValueError("kcache must be (batch, capacity, heads, head_dim)")
    _, cap, Hkv, dk = kcache.shape
    if dk != d or tuple(vcache.shape) != tuple(kcache.shape) or kcache.shape[0] != B:
        raise ValueError("cache shapes do not match q")
    for t, n in ((q, "q"), (kcache, "kcache"), (vcache, "vcache")):
        _check(t, n, torch.bfloat16, q.device)
    _check(cache_seqlens, "cache_seqlens", torch.int32, q.device)
    _shape(cache_seqlens, (B,), "cache_seqlens")
    if num_splits is None:
        num_splits = fa_kvcache_default_splits(B, Hkv, cap, d)
    if o is None:
        o = torch.empty_like(q)
    _check(o, "o", torch.bfloat16, q.device)
    _shape(o, q.shape, "o")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, q.device)
        _shape(lse, (B, Hq), "lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_kvcache_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(cache_seqlens), _ptr(o), _ptr(lse),
                                      int(num_splits), B, Hq, Hkv, cap, d, float(scale), _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_kvcache_noalloc")
    return o, lse


def fa_fwd_kvcache_paged(q, kpages, vpages, block_table, cache_seqlens, o=None, lse=None, num_splits=None,
                         scale=None, workspace=None, stream=None, want_lse=True):
    """Split-KV decode over a paged cache through ``fa_fwd_kvcache_paged``.

    q: (B, 1, Hq, d) bf16; kpages, vpages: (num_pages, page_size, Hkv, d)
    bf16; block_table: (B, pages_per_seq) int32; cache_seqlens: (B,) int32,
    all on one GPU. Returns (o (B, 1, Hq, d) bf16, lse (B, Hq) float32).
    """
    import torch
    if q.dim() != 4 or q.shape[1] != 1:
        raise ValueError("q must be (batch, 1, heads, head_dim)")
    B, _, Hq, d = q.shape
    num_pages, page_size, Hkv, dk = kpages.shape
    if dk != d or tuple(vpages.shape) != tuple(kpages.shape):
        raise ValueError("page pool shapes do not match q")
    for t, n in ((q, "q"), (kpages, "kpages"), (vpages, "vpages")):
        _check(t, n, torch.bfloat16, q.device)
    _check(block_table, "block_table", torch.int32, q.device)
    _check(cache_seqlens, "cache_seqlens", torch.int32, q.device)
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(cache_seqlens.shape) != (B,):
        raise ValueError("block_table must be (B, pages_per_seq) and cache_seqlens (B,)")
    pages_per_seq = block_table.shape[1]
    if num_splits is None:
        num_splits = fa_kvcache_default_splits(B, Hkv, page_size * pages_per_seq, d)
    if o is None:
        o = torch.empty_like(q)
    _check(o, "o", torch.bfloat16, q.device)
    _shape(o, q.shape, "o")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, q.device)
        _shape(lse, (B, Hq), "lse")
    workspace, ws_bytes = _workspace(workspace, fa_fwd_kvcache_workspace_size(B, Hq, d, num_splits), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_kvcache_paged(_ptr(q), _ptr(kpages), _ptr(vpages), _ptr(block_table), _ptr(cache_seqlens),
                                    _ptr(o), _ptr(lse), int(num_splits), B, Hq, Hkv, page_size, pages_per_seq,
                                    num_pages, d, float(scale), _ptr(workspace), ws_bytes, _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_kvcache_paged")
    return o, lse


def _append_common(q, k_new, v_new, cache_seqlens, Hkv, d, cap, o, lse, num_splits, workspace, want_lse):
    import torch
    if q.dim() != 4:
        raise ValueError("q must be (batch, queries, heads, head_dim)")
    B, Nq, Hq, dq = q.shape
    if dq != d:
        raise ValueError("cache head_dim does not match q")
    _check(q, "q", torch.bfloat16, q.device)
    if (k_new is None) != (v_new is None):
        raise ValueError("give both k_new and v_new, or neither")
    if k_new is not None:
        for t, n in ((k_new, "k_new"), (v_new, "v_new")):
            _check(t, n, torch.bfloat16, q.device)
            if tuple(t.shape) != (B, Nq, Hkv, d):
                raise ValueError(f"{n} must be (B, Nq, Hkv, d)")
    _check(cache_seqlens, "cache_seqlens", torch.int32, q.device)
    if tuple(cache_seqlens.shape) != (B,):
        raise ValueError("cache_seqlens must be (B,)")
    if num_splits is None:
        num_splits = (fa_kvcache_default_splits(B, Hkv, cap, d) if Nq == 1 and k_new is None
                      else fa_kvcache_append_default_splits(B, Nq, Hkv, Hq, cap, d))
    if o is None:
        o = torch.empty_like(q)
    _check(o, "o", torch.bfloat16, q.device)
    _shape(o, q.shape, "o")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, q.device)
        _shape(lse, (B, Hq, Nq), "lse")
    workspace, ws_bytes = _workspace(workspace, fa_fwd_kvcache_workspace_size(B * Nq, Hq, d, num_splits), q.device)
    return B, Nq, Hq, o, lse, int(num_splits), workspace, ws_bytes


def fa_fwd_kvcache_append(q, kcache, vcache, cache_seqlens, k_new=None, v_new=None, causal=True, o=None, lse=None,
                          num_splits=None, scale=None, workspace=None, stream=None, want_lse=True):
    """Decode step with in-place cache append through ``fa_fwd_kvcache_append``.

    q: (B, Nq, Hq, d) bf16; kcache, vcache: (B, capacity, Hkv, d) bf16,
    written in place at rows cache_seqlens[b] .. + Nq - 1 when k_new, v_new
    (B, Nq, Hkv, d) are given; cache_seqlens: (B,) int32, not advanced.
    Returns (o (B, Nq, Hq, d) bf16, lse (B, Hq, Nq) float32).
    """
    import torch
    if q.dim() != 4 or kcache.dim() != 4:
        raise ValueError("q must be (batch, queries, heads, head_dim) and the caches (batch, capacity, heads, "
                         "head_dim)")
    _, cap, Hkv, d = kcache.shape
    if tuple(vcache.shape) != tuple(kcache.shape) or kcache.shape[0] != q.shape[0]:
        raise ValueError("cache shapes do not match q")
    for t, n in ((kcache, "kcache"), (vcache, "vcache")):
        _check(t, n, torch.bfloat16, q.device)
    B, Nq, Hq, o, lse, S, workspace, ws_bytes = _append_common(q, k_new, v_new, cache_seqlens, Hkv, d, cap, o, lse,
                                                                num_splits, workspace, want_lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_kvcache_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kcache), _ptr(vcache),
                                     _ptr(cache_seqlens), _ptr(o), _ptr(lse), int(bool(causal)), S, B, Nq, Hq, Hkv,
                                     cap, d, float(scale), _ptr(workspace), ws_bytes, _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_kvcache_append")
    return o, lse


def fa_fwd_kvcache_paged_append(q, kpages, vpages, block_table, cache_seqlens, k_new=None, v_new=None, causal=True,
                                o=None, lse=None, num_splits=None, scale=None, workspace=None, stream=None,
                                want_lse=True):
    """``fa_fwd_kvcache_append`` over a paged cache (``fa_fwd_kvcache_paged_append``).

    kpages, vpages: (num_pages, page_size, Hkv, d) bf16; block_table:
    (B, pages_per_seq) int32. Returns (o (B, Nq, Hq, d), lse (B, Hq, Nq)).
    """
    import torch
    num_pages, page_size, Hkv, d = kpages.shape
    if tuple(vpages.shape) != tuple(kpages.shape):
        raise ValueError("page pool shapes do not match")
    for t, n in ((kpages, "kpages"), (vpages, "vpages")):
        _check(t, n, torch.bfloat16, q.device)
    _check(block_table, "block_table", torch.int32, q.device)
    if block_table.dim() != 2 or block_table.shape[0] != q.shape[0]:
        raise ValueError("block_table must be (B, pages_per_seq)")
    pages_per_seq = block_table.shape[1]
    B, Nq, Hq, o, lse, S, workspace, ws_bytes = _append_common(q, k_new, v_new, cache_seqlens, Hkv, d,
                                                                page_size * pages_per_seq, o, lse, num_splits,
                                                                workspace, want_lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_kvcache_paged_append(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(kpages), _ptr(vpages),
                                           _ptr(block_table), _ptr(cache_seqlens), _ptr(o), _ptr(lse),
                                           int(bool(causal)), S, B, Nq, Hq, Hkv, page_size, pages_per_seq, num_pages,
                                           d, float(scale), _ptr(workspace), ws_bytes, _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_kvcache_paged_append")
    return o, lse


def fa_fp8_padded_rows(n):
    return int(lib().fa_fp8_padded_rows(int(n)))


def fa_quantize_fp8(x, signs=None, transpose=False, codes=None, scales=None, stream=None):
    """Block quantisation to e4m3 through ``fa_quantize_fp8``.

    x: (B, N, H, d) bf16; signs: (d,) float32 of +-1 (rotation) or None.
    Returns (codes uint8 (B, H, Np, d), or (B, H, d, Np) when transpose,
    scales uint8 (B, H, Np / 64)), Np = fa_fp8_padded_rows(N).
    """
    import torch
    if x.dim() != 4:
        raise ValueError("x must be (batch, seq, heads, head_dim)")
    B, N, H, d = x.shape
    _check(x, "x", torch.bfloat16, x.device)
    if signs is not None:
        _check(signs, "signs", torch.float32, x.device)
        if tuple(signs.shape) != (d,):
            raise ValueError("signs must be (head_dim,)")
    Np = fa_fp8_padded_rows(N)
    shape = (B, H, d, Np) if transpose else (B, H, Np, d)
    if codes is None:
        codes = torch.empty(shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, Np // 64), dtype=torch.uint8, device=x.device)
    _check(codes, "codes", torch.uint8, x.device)
    _check(scales, "scales", torch.uint8, x.device)
    if tuple(codes.shape) != shape or tuple(scales.shape) != (B, H, Np // 64):
        raise ValueError("codes / scales have the wrong shape")
    st = lib().fa_quantize_fp8(_ptr(x), _ptr(signs), _ptr(codes), _ptr(scales), int(bool(transpose)), B, N, H, d,
                               _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_quantize_fp8")
    return codes, scales


def fa_fwd_fp8(q8, q_scales, k8, k_scales, vt8, v_scales, Nq, Nk, causal=False, scale=None, o=None, lse=None,
               stream=None, want_lse=True):
    """Attention on e4m3 operands through ``fa_fwd_fp8``.

    q8 (B, Hq, Nqp, d), k8 (B, Hkv, Nkp, d), vt8 (B, Hkv, d, Nkp) uint8 codes
    and their (.., Np / 64) uint8 scales as ``fa_quantize_fp8`` returns
    them; Nq, Nk the unpadded lengths. Returns (o (B, Nq, Hq, d) bf16,
    lse (B, Hq, Nq) float32).
    """
    import torch
    B, Hq, Nqp, d = q8.shape
    Hkv = k8.shape[1]
    if Nqp != fa_fp8_padded_rows(Nq) or tuple(k8.shape) != (B, Hkv, fa_fp8_padded_rows(Nk), d) \
            or tuple(vt8.shape) != (B, Hkv, d, fa_fp8_padded_rows(Nk)):
        raise ValueError("code tensors do not match Nq / Nk")
    for t, n in ((q8, "q8"), (k8, "k8"), (vt8, "vt8"), (q_scales, "q_scales"), (k_scales, "k_scales"),
                 (v_scales, "v_scales")):
        _check(t, n, torch.uint8, q8.device)
    _shape(q_scales, (B, Hq, Nqp // 64), "q_scales")
    _shape(k_scales, (B, Hkv, fa_fp8_padded_rows(Nk) // 64), "k_scales")
    _shape(v_scales, (B, Hkv, fa_fp8_padded_rows(Nk) // 64), "v_scales")
    if o is None:
        o = torch.empty((B, Nq, Hq, d), dtype=torch.bfloat16, device=q8.device)
    _check(o, "o", torch.bfloat16, q8.device)
    _shape(o, (B, Nq, Hq, d), "o")
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q8.device)
    if lse is not None:
        _check(lse, "lse", torch.float32, q8.device)
        _shape(lse, (B, Hq, Nq), "lse")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_fwd_fp8(_ptr(q8), _ptr(q_scales), _ptr(k8), _ptr(k_scales), _ptr(vt8), _ptr(v_scales), _ptr(o),
                          _ptr(lse), B, Hq, Hkv, int(Nq), int(Nk), d, int(bool(causal)), float(scale),
                          _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_fp8")
    return o, lse


def fa_bwd_workspace_size(B, Hq, Nq):
    return int(lib().fa_bwd_workspace_size(int(B), int(Hq), int(Nq)))


def fa_bwd(q, k, v, o, lse, dout, causal=False, scale=None, dq=None, dk=None, dv=None, workspace=None,
           stream=None):
    """Attention backward through ``fa_bwd``.

    q, o, dout: (B, Nq, Hq, d) bf16; k, v: (B, Nk, Hkv, d) bf16; lse:
    (B, Hq, Nq) float32 from the forward. Gradient tensors and the
    workspace are allocated when not given. Returns (dq, dk, dv).
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be (batch, seq, heads, head_dim)")
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Nk, Hkv, d) or tuple(v.shape) != (B, Nk, Hkv, d):
        raise ValueError("k/v shapes do not match q")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check(t, n, torch.bfloat16, q.device)
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    _check(lse, "lse", torch.float32, q.device)
    if tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("lse must be (B, Hq, Nq)")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _check(t, n, torch.bfloat16, q.device)
        if tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"{n} must have the shape of {n[1:]}")
    workspace, ws_bytes = _workspace(workspace, fa_bwd_workspace_size(B, Hq, Nq), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                      B, Hq, Hkv, Nq, Nk, d, int(bool(causal)), float(scale), _ptr(workspace), ws_bytes,
                      _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv


def fa_bwd_window(q, k, v, o, lse, dout, window_left, window_right, scale=None, dq=None, dk=None, dv=None,
                  workspace=None, stream=None):
    """Attention backward under a bottom-right aligned window through
    ``fa_bwd_window``; shapes as ``fa_bwd``. Returns (dq, dk, dv)."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be (batch, seq, heads, head_dim)")
    B, Nq, Hq, d = q.shape
    _, Nk, Hkv, _ = k.shape
    if tuple(k.shape) != (B, Nk, Hkv, d):
        raise ValueError("k does not match q")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, n, torch.bfloat16, q.device)
    for t, n in ((o, "o"), (dout, "dout"), (dq, "dq")):
        _shape(t, q.shape, n)
    for t, n in ((v, "v"), (dk, "dk"), (dv, "dv")):
        _shape(t, k.shape, n)
    _check(lse, "lse", torch.float32, q.device)
    _shape(lse, (B, Hq, Nq), "lse")
    workspace, ws_bytes = _workspace(workspace, fa_bwd_workspace_size(B, Hq, Nq), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_bwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                             _ptr(dv), B, Hq, Hkv, Nq, Nk, d, int(window_left), int(window_right), float(scale),
                             _ptr(workspace), ws_bytes, _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_window")
    return dq, dk, dv


def fa_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, window_left=-1,
                  window_right=-1, scale=None, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Attention backward over a packed batch through ``fa_bwd_varlen``:
    q, o, dout (total_q, Hq, d), k, v (total_k, Hkv, d) bf16, lse (Hq,
    total_q) float32 as ``fa_fwd_varlen`` returns it. Returns (dq, dk, dv)."""
    import torch
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q, k, v must be (tokens, heads, head_dim)")
    total_q, Hq, d = q.shape
    total_k, Hkv, _ = k.shape
    if k.shape[2] != d:
        raise ValueError("k does not match q")
    B = cu_seqlens_q.shape[0] - 1
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check(t, n, torch.bfloat16, q.device)
    for t, n in ((o, "o"), (dout, "dout"), (dq, "dq")):
        _shape(t, q.shape, n)
    for t, n in ((v, "v"), (dk, "dk"), (dv, "dv")):
        _shape(t, k.shape, n)
    _check(lse, "lse", torch.float32, q.device)
    _shape(lse, (Hq, total_q), "lse")
    _check(cu_seqlens_q, "cu_seqlens_q", torch.int32, q.device)
    _check(cu_seqlens_k, "cu_seqlens_k", torch.int32, q.device)
    if B < 0 or cu_seqlens_q.dim() != 1 or tuple(cu_seqlens_k.shape) != (B + 1,):
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be (B + 1,)")
    workspace, ws_bytes = _workspace(workspace, fa_bwd_workspace_size(B, Hq, max_seqlen_q), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                             _ptr(dv), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Hq, Hkv, int(max_seqlen_q),
                             int(max_seqlen_k), total_q, total_k, d, int(window_left), int(window_right),
                             float(scale), _ptr(workspace), ws_bytes, _stream(stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_varlen")
    return dq, dk, dv
