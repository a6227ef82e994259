"""Exact tiled attention on AMD Instinct MI355X (gfx950): Python binding of libfa.so.

The binding only marshals arguments: it checks tensor shapes, dtypes, devices and
contiguity, allocates outputs with PyTorch when the caller passes none, and calls the
C ABI declared in ``include/fa.h`` through ctypes on the current HIP stream. Every step
of the computation runs in the library's HIP kernels; there is no fallback. If the
library is not built, every entry point raises.

Entry points (same names as the C ABI):
    fa_fwd(q, k, v, scale, causal=False, kv_len=None, o=None, lse=None) -> (o, lse)
    fa_fwd_blocksparse(q, k, v, scale, block_mask, mask_block=128, causal=False,
                       kv_len=None, o=None, lse=None) -> (o, lse)
    fa_fwd_dropout(q, k, v, scale, dropout_p, seed, causal=False, kv_len=None, o=None,
                   lse=None) -> (o, lse)
    fa_bwd_dropout(q, k, v, o, dout, lse, scale, dropout_p, seed, causal=False, kv_len=None,
                   dq=None, dk=None, dv=None, workspace=None) -> (dq, dk, dv)
    fa_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, scale, causal=False, window_left=-1,
                  window_right=-1, o=None, lse=None) -> (o, lse)
    fa_bwd_varlen_workspace_bytes(H, total, d) -> int
    fa_bwd_varlen(q, k, v, o, dout, lse, cu_seqlens, max_seqlen, scale, causal=False,
                  window_left=-1, window_right=-1, dq=None, dk=None, dv=None,
                  workspace=None) -> (dq, dk, dv)
    fa_fwd_kvcache_workspace_bytes(B, H, Nq, Nk, d) -> int
    fa_fwd_kvcache(q, k_cache, v_cache, scale, causal=False, kv_len=None, o=None, lse=None,
                   workspace=None) -> (o, lse)
    fa_fwd_kvcache_noalloc(q, k_cache, v_cache, scale, o, lse, causal=False, kv_len=None)
        -> (o, lse)   (partial results in the library's static scratch; o, lse required)
    fa_bwd_workspace_bytes(B, H, N, d) -> int
    fa_bwd(q, k, v, o, dout, lse, scale, causal=False, kv_len=None, block_mask=None,
           mask_block=128, dq=None, dk=None, dv=None, workspace=None) -> (dq, dk, dv)
    fa_status_string(status) -> str
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "FA_F32", "FA_BF16", "FA_OK", "FA_ERR_INVALID", "FA_ERR_UNSUPPORTED", "FA_ERR_HIP",
    "FAError", "lib_path", "load", "fa_fwd", "fa_fwd_blocksparse", "fa_bwd",
    "fa_bwd_workspace_bytes", "fa_fwd_dropout", "fa_bwd_dropout", "fa_fwd_varlen", "fa_bwd_varlen", "fa_bwd_varlen_workspace_bytes", "fa_fwd_kvcache", "fa_fwd_kvcache_workspace_bytes", "fa_fwd_kvcache_noalloc", "NOALLOC_SCRATCH_BYTES", "fa_time_next_call", "fa_status_string", "EXPORTED_SYMBOLS",
]

FA_F32, FA_BF16 = 0, 1
FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3

EXPORTED_SYMBOLS = ("fa_fwd", "fa_fwd_blocksparse", "fa_bwd_workspace_bytes", "fa_bwd",
                    "fa_fwd_kvcache_workspace_bytes", "fa_fwd_kvcache", "fa_fwd_kvcache_noalloc",
                    "fa_fwd_varlen", "fa_bwd_varlen_workspace_bytes", "fa_bwd_varlen",
                    "fa_fwd_dropout", "fa_bwd_dropout",
                    "fa_time_next_call", "fa_status_string", "fa_last_error")

_LIB = None
NOALLOC_SCRATCH_BYTES = 64 << 20  # FA_NOALLOC_SCRATCH_BYTES of include/fa.h


class FAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")


def load() -> ctypes.CDLL:
    """Load libfa.so once. Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"HIP attention library missing: {path} (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [I, I, I, I, I, P, P, P, P, P, F, I, P, P]
    lib.fa_fwd.restype = I
    lib.fa_fwd_blocksparse.argtypes = [I, I, I, I, I, P, P, P, P, P, F, I, P, P, I, P]
    lib.fa_fwd_blocksparse.restype = I
    lib.fa_bwd_workspace_bytes.argtypes = [I, I, I, I]
    lib.fa_bwd_workspace_bytes.restype = S
    lib.fa_bwd.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, F, I, P, P, I, P, S, P]
    lib.fa_bwd.restype = I
    U64 = ctypes.c_uint64
    lib.fa_fwd_dropout.argtypes = [I, I, I, I, I, P, P, P, P, P, F, I, P, F, U64, P]
    lib.fa_fwd_dropout.restype = I
    lib.fa_bwd_dropout.argtypes = [I, I, I, I, I, P, P, P, P, P, P, P, P, P, F, I, P, F, U64, P, S, P]
    lib.fa_bwd_dropout.restype = I
    lib.fa_fwd_varlen.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, F, I, I, I, P]
    lib.fa_fwd_varlen.restype = I
    lib.fa_bwd_varlen_workspace_bytes.argtypes = [I, I, I]
    lib.fa_bwd_varlen_workspace_bytes.restype = S
    lib.fa_bwd_varlen.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, F, I, I, I, P, S, P]
    lib.fa_bwd_varlen.restype = I
    lib.fa_fwd_kvcache_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.fa_fwd_kvcache_workspace_bytes.restype = S
    lib.fa_fwd_kvcache.argtypes = [I, I, I, I, I, I, P, P, P, P, P, F, I, P, P, S, P]
    lib.fa_fwd_kvcache.restype = I
    lib.fa_fwd_kvcache_noalloc.argtypes = [I, I, I, I, I, I, P, P, P, P, P, F, I, P, P]
    lib.fa_fwd_kvcache_noalloc.restype = I
    lib.fa_status_string.argtypes = [I]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_time_next_call.argtypes = [P, I]
    lib.fa_time_next_call.restype = None
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def fa_time_next_call(events) -> None:
    """Measurement hook: the next call on this thread records events[0] on its stream before
    its first kernel and events[i] after its i-th kernel (timing-enabled torch.cuda.Event
    objects that have been recorded once, so that their HIP events exist; at most 8). Pass
    None or [] to clear."""
    lib = load()
    if not events:
        lib.fa_time_next_call(None, 0)
        return
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e.cuda_event) for e in events])
    lib.fa_time_next_call(arr, len(events))


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != FA_OK:
        lib = load()
        raise FAError(status, f"{lib.fa_status_string(status).decode()}: {lib.fa_last_error().decode()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _dev_tensor(t: torch.Tensor, name: str, like: torch.Tensor | None = None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous ([B, H, N, d] row-major)")
    if like is not None and (t.shape != like.shape or t.dtype != like.dtype or t.device != like.device):
        raise ValueError(f"{name} must match q in shape, dtype and device")
    return t


def _f32_out(t, name: str, shape, q: torch.Tensor) -> torch.Tensor:
    """A caller-supplied fp32 output (lse): device tensor on q's device, given shape."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != q.device:
        raise ValueError(f"{name} must be a device tensor on {q.device}")
    if tuple(t.shape) != tuple(shape) or t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor {list(shape)}")
    return t


def _workspace(ws, need: int, q: torch.Tensor) -> torch.Tensor:
    """The caller's workspace, or a new one of `need` bytes: a uint8 device tensor on q's
    device (its size is checked by the library)."""
    if ws is None:
        return torch.empty(max(int(need), 1), dtype=torch.uint8, device=q.device)
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != q.device:
        raise ValueError(f"workspace must be a device tensor on {q.device}")
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    return ws


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _kv_len(kv_len, q):
    if kv_len is None:
        return None
    kv = _dev_tensor(kv_len, "kv_len")
    if kv.dtype != torch.int32 or kv.shape != (q.shape[0],) or kv.device != q.device:
        raise ValueError("kv_len must be an int32 device tensor of shape [B]")
    return kv


def _mask(block_mask, q, mask_block):
    if block_mask is None:
        return None
    m = _dev_tensor(block_mask, "block_mask")
    nb = -(-q.shape[2] // int(mask_block)) if mask_block > 0 else 0
    if m.dtype != torch.uint8 or m.shape != (nb, nb) or m.device != q.device:
        raise ValueError(f"block_mask must be a uint8 device tensor of shape [{nb}, {nb}]")
    return m


def _fwd_common(q, k, v, o, lse):
    q = _dev_tensor(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    _dev_tensor(k, "k", q)
    _dev_tensor(v, "v", q)
    B, H, N, d = q.shape
    o = torch.empty_like(q) if o is None else _dev_tensor(o, "o", q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        _f32_out(lse, "lse", (B, H, N), q)
    return q, o, lse


def fa_fwd(q, k, v, scale: float, causal: bool = False, kv_len=None, o=None, lse=None):
    """O and lse (natural log) of exact attention; see ``fa_fwd`` in include/fa.h."""
    lib = load()
    q, o, lse = _fwd_common(q, k, v, o, lse)
    kv = _kv_len(kv_len, q)
    B, H, N, d = q.shape
    _check(lib.fa_fwd(_dtype_code(q), B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                      float(scale), int(bool(causal)), _ptr(kv), _stream(q.device)))
    return o, lse


def fa_fwd_blocksparse(q, k, v, scale: float, block_mask, mask_block: int = 128, causal: bool = False,
                       kv_len=None, o=None, lse=None):
    """Block-sparse forward; see ``fa_fwd_blocksparse`` in include/fa.h."""
    lib = load()
    q, o, lse = _fwd_common(q, k, v, o, lse)
    kv = _kv_len(kv_len, q)
    m = _mask(block_mask, q, mask_block)
    if m is None:
        raise ValueError("block_mask is required")
    B, H, N, d = q.shape
    _check(lib.fa_fwd_blocksparse(_dtype_code(q), B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                  _ptr(lse), float(scale), int(bool(causal)), _ptr(kv), _ptr(m),
                                  int(mask_block), _stream(q.device)))
    return o, lse


def fa_bwd_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load().fa_bwd_workspace_bytes(int(B), int(H), int(N), int(d)))


def fa_bwd(q, k, v, o, dout, lse, scale: float, causal: bool = False, kv_len=None, block_mask=None,
           mask_block: int = 128, dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV; see ``fa_bwd`` in include/fa.h. ``workspace`` is a uint8 device tensor."""
    lib = load()
    q = _dev_tensor(q, "q")
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _dev_tensor(t, name, q)
    B, H, N, d = q.shape
    _f32_out(lse, "lse", (B, H, N), q)
    dq = torch.empty_like(q) if dq is None else _dev_tensor(dq, "dq", q)
    dk = torch.empty_like(q) if dk is None else _dev_tensor(dk, "dk", q)
    dv = torch.empty_like(q) if dv is None else _dev_tensor(dv, "dv", q)
    kv = _kv_len(kv_len, q)
    m = _mask(block_mask, q, mask_block)
    workspace = _workspace(workspace, fa_bwd_workspace_bytes(B, H, N, d), q)
    _check(lib.fa_bwd(_dtype_code(q), B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                      _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), float(scale), int(bool(causal)), _ptr(kv),
                      _ptr(m), int(mask_block), _ptr(workspace), int(workspace.numel()),
                      _stream(q.device)))
    return dq, dk, dv


def fa_fwd_kvcache_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int) -> int:
    return int(load().fa_fwd_kvcache_workspace_bytes(int(B), int(H), int(Nq), int(Nk), int(d)))


def fa_fwd_kvcache(q, k_cache, v_cache, scale: float, causal: bool = False, kv_len=None, o=None,
                   lse=None, workspace=None):
    """Queries [B, H, Nq, d] against a key/value cache [B, H, Nk, d]; see ``fa_fwd_kvcache``
    in include/fa.h. ``workspace`` is a uint8 device tensor."""
    lib = load()
    q = _dev_tensor(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d]")
    k_cache = _dev_tensor(k_cache, "k_cache")
    _dev_tensor(v_cache, "v_cache", k_cache)
    B, H, Nq, d = q.shape
    Nk = k_cache.shape[2]
    if (k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[1] != H or k_cache.shape[3] != d
            or k_cache.dtype != q.dtype or k_cache.device != q.device):
        raise ValueError("k_cache and v_cache must be [B, H, Nk, d] of q's dtype and device")
    o = torch.empty_like(q) if o is None else _dev_tensor(o, "o", q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    else:
        _f32_out(lse, "lse", (B, H, Nq), q)
    kv = _kv_len(kv_len, q)
    workspace = _workspace(workspace, fa_fwd_kvcache_workspace_bytes(B, H, Nq, Nk, d), q)
    _check(lib.fa_fwd_kvcache(_dtype_code(q), B, H, Nq, Nk, d, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                              _ptr(o), _ptr(lse), float(scale), int(bool(causal)), _ptr(kv),
                              _ptr(workspace), int(workspace.numel()), _stream(q.device)))
    return o, lse


def fa_fwd_kvcache_noalloc(q, k_cache, v_cache, scale: float, o, lse, causal: bool = False, kv_len=None):
    """The cache forward without a workspace: its partial results live in the library's
    static device scratch (see ``fa_fwd_kvcache_noalloc`` in include/fa.h). The outputs o
    [B, H, Nq, d] and lse [B, H, Nq] are the caller's; nothing is allocated here either."""
    lib = load()
    q = _dev_tensor(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d]")
    k_cache = _dev_tensor(k_cache, "k_cache")
    _dev_tensor(v_cache, "v_cache", k_cache)
    B, H, Nq, d = q.shape
    Nk = k_cache.shape[2]
    if (k_cache.dim() != 4 or k_cache.shape[0] != B or k_cache.shape[1] != H or k_cache.shape[3] != d
            or k_cache.dtype != q.dtype or k_cache.device != q.device):
        raise ValueError("k_cache and v_cache must be [B, H, Nk, d] of q's dtype and device")
    if o is None or lse is None:
        raise ValueError("o and lse are required (this call allocates nothing)")
    _dev_tensor(o, "o", q)
    _f32_out(lse, "lse", (B, H, Nq), q)
    kv = _kv_len(kv_len, q)
    _check(lib.fa_fwd_kvcache_noalloc(_dtype_code(q), B, H, Nq, Nk, d, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(o), _ptr(lse), float(scale), int(bool(causal)), _ptr(kv),
                                      _stream(q.device)))
    return o, lse


def _cu_seqlens(cu_seqlens, q):
    cu = _dev_tensor(cu_seqlens, "cu_seqlens")
    if cu.dtype != torch.int32 or cu.dim() != 1 or cu.numel() < 2 or cu.device != q.device:
        raise ValueError("cu_seqlens must be an int32 device tensor of shape [nseq + 1]")
    return cu


def _packed(q):
    q = _dev_tensor(q, "q")
    if q.dim() != 3:
        raise ValueError("packed tensors are [total, H, d]")
    return q


def fa_fwd_varlen(q, k, v, cu_seqlens, max_seqlen: int, scale: float, causal: bool = False,
                  window_left: int = -1, window_right: int = -1, o=None, lse=None):
    """Packed variable-length forward; see ``fa_fwd_varlen`` in include/fa.h. q, k, v are
    [total, H, d]; returns o [total, H, d] and lse [H, total]."""
    lib = load()
    q = _packed(q)
    _dev_tensor(k, "k", q)
    _dev_tensor(v, "v", q)
    cu = _cu_seqlens(cu_seqlens, q)
    total, H, d = q.shape
    o = torch.empty_like(q) if o is None else _dev_tensor(o, "o", q)
    if lse is None:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    else:
        _f32_out(lse, "lse", (H, total), q)
    _check(lib.fa_fwd_varlen(_dtype_code(q), cu.numel() - 1, H, total, int(max_seqlen), d, _ptr(cu), _ptr(q),
                             _ptr(k), _ptr(v), _ptr(o), _ptr(lse), float(scale), int(bool(causal)),
                             int(window_left), int(window_right), _stream(q.device)))
    return o, lse


def fa_bwd_varlen_workspace_bytes(H: int, total: int, d: int) -> int:
    return int(load().fa_bwd_varlen_workspace_bytes(int(H), int(total), int(d)))


def fa_bwd_varlen(q, k, v, o, dout, lse, cu_seqlens, max_seqlen: int, scale: float, causal: bool = False,
                  window_left: int = -1, window_right: int = -1, dq=None, dk=None, dv=None, workspace=None):
    """Backward of ``fa_fwd_varlen``; see ``fa_bwd_varlen`` in include/fa.h."""
    lib = load()
    q = _packed(q)
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _dev_tensor(t, name, q)
    cu = _cu_seqlens(cu_seqlens, q)
    total, H, d = q.shape
    _f32_out(lse, "lse", (H, total), q)
    dq = torch.empty_like(q) if dq is None else _dev_tensor(dq, "dq", q)
    dk = torch.empty_like(q) if dk is None else _dev_tensor(dk, "dk", q)
    dv = torch.empty_like(q) if dv is None else _dev_tensor(dv, "dv", q)
    workspace = _workspace(workspace, fa_bwd_varlen_workspace_bytes(H, total, d), q)
    _check(lib.fa_bwd_varlen(_dtype_code(q), cu.numel() - 1, H, total, int(max_seqlen), d, _ptr(cu), _ptr(q),
                             _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                             float(scale), int(bool(causal)), int(window_left), int(window_right),
                             _ptr(workspace), int(workspace.numel()), _stream(q.device)))
    return dq, dk, dv


def fa_fwd_dropout(q, k, v, scale: float, dropout_p: float, seed: int, causal: bool = False, kv_len=None,
                   o=None, lse=None):
    """Forward with dropout on the probabilities; see ``fa_fwd_dropout`` in include/fa.h."""
    lib = load()
    q, o, lse = _fwd_common(q, k, v, o, lse)
    kv = _kv_len(kv_len, q)
    B, H, N, d = q.shape
    _check(lib.fa_fwd_dropout(_dtype_code(q), B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              float(scale), int(bool(causal)), _ptr(kv), float(dropout_p),
                              int(seed) & 0xFFFFFFFFFFFFFFFF, _stream(q.device)))
    return o, lse


def fa_bwd_dropout(q, k, v, o, dout, lse, scale: float, dropout_p: float, seed: int, causal: bool = False,
                   kv_len=None, dq=None, dk=None, dv=None, workspace=None):
    """Backward of ``fa_fwd_dropout`` (same dropout_p and seed); see include/fa.h."""
    lib = load()
    q = _dev_tensor(q, "q")
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _dev_tensor(t, name, q)
    B, H, N, d = q.shape
    _f32_out(lse, "lse", (B, H, N), q)
    dq = torch.empty_like(q) if dq is None else _dev_tensor(dq, "dq", q)
    dk = torch.empty_like(q) if dk is None else _dev_tensor(dk, "dk", q)
    dv = torch.empty_like(q) if dv is None else _dev_tensor(dv, "dv", q)
    kv = _kv_len(kv_len, q)
    workspace = _workspace(workspace, fa_bwd_workspace_bytes(B, H, N, d), q)
    _check(lib.fa_bwd_dropout(_dtype_code(q), B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                              _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), float(scale), int(bool(causal)), _ptr(kv),
                              float(dropout_p), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(workspace),
                              int(workspace.numel()), _stream(q.device)))
    return dq, dk, dv
