"""Host-side tests of the C ABI: the library loads, exports what include/fa.h declares,
sizes its workspace linearly in N, and rejects invalid requests before touching a device.

No call here reaches a kernel launch: every request fails validation on the host, so
the tests run without a GPU (fake, well-aligned pointer values are never dereferenced).
"""
import ctypes
import os
import re

import pytest

import exact_tiled_attention_32_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.lib_path()):
        from exact_tiled_attention_32_amd import build
        build.build(verbose=False)
    return fa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(fa.EXPORTED_SYMBOLS), names
    for n in names:
        assert getattr(lib, n) is not None


def test_workspace_bytes_linear_in_n(lib):
    # exact formula: align256(rows * 4) + 4 KiB: the fp32 D = rowsum(dO * O) of every row,
    # then the block-sparse key-tile order (1024 entries)
    for B, H, N, d in [(1, 1, 1, 64), (8, 16, 512, 64), (1, 16, 16384, 128), (1, 8, 65536, 64)]:
        rows = B * H * N
        al = lambda x: (x + 255) // 256 * 256
        assert fa.fa_bwd_workspace_bytes(B, H, N, d) == al(rows * 4) + 4096
    # O(N): doubling N doubles the workspace (no N^2 term)
    ws = lambda n: fa.fa_bwd_workspace_bytes(1, 1, n, 64) - 4096
    assert ws(32768) == 2 * ws(16384)
    assert fa.fa_bwd_workspace_bytes(0, 1, 1, 64) == 0
    assert fa.fa_bwd_workspace_bytes(1, 1, -5, 64) == 0


def test_status_strings(lib):
    for s in (fa.FA_OK, fa.FA_ERR_INVALID, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_HIP):
        assert fa.fa_status_string(s).startswith("FA_")
    assert fa.fa_status_string(99) == "unknown fa_status"


P = 0x10000  # fake, 256-byte aligned device address; never dereferenced


def fwd(lib, dt=fa.FA_BF16, B=1, H=1, N=128, d=64, q=P, k=P, v=P, o=P, lse=P, scale=0.125,
        causal=0, kv_len=None):
    c = ctypes.c_void_p
    return lib.fa_fwd(dt, B, H, N, d, c(q), c(k), c(v), c(o), c(lse), scale, causal,
                      None if kv_len is None else c(kv_len), None)


def fwd_sparse(lib, mask=P, mb=128, **kw):
    c = ctypes.c_void_p
    return lib.fa_fwd_blocksparse(kw.get("dt", fa.FA_BF16), 1, 1, kw.get("N", 256), 64, c(P), c(P), c(P),
                                  c(P), c(P), 0.125, 0, None, None if mask is None else c(mask), mb, None)


def bwd(lib, dt=fa.FA_BF16, N=128, d=64, ws=P, ws_bytes=None, mask=None, mb=128, dq=P, scale=0.125):
    c = ctypes.c_void_p
    need = fa.fa_bwd_workspace_bytes(1, 1, N, d) if ws_bytes is None else ws_bytes
    return lib.fa_bwd(dt, 1, 1, N, d, c(P), c(P), c(P), c(P), c(P), c(P), c(dq), c(P), c(P), scale, 0, None,
                      None if mask is None else c(mask), mb, None if ws is None else c(ws), need, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(q=0), fa.FA_ERR_INVALID),
    (dict(o=0), fa.FA_ERR_INVALID),
    (dict(lse=0), fa.FA_ERR_INVALID),
    (dict(k=P + 8), fa.FA_ERR_INVALID),          # not 16-byte aligned
    (dict(lse=P + 2), fa.FA_ERR_INVALID),        # not 4-byte aligned
    (dict(kv_len=P + 1), fa.FA_ERR_INVALID),
    (dict(B=0), fa.FA_ERR_INVALID),
    (dict(N=-3), fa.FA_ERR_INVALID),
    (dict(H=1 << 30, N=1 << 30), fa.FA_ERR_INVALID),  # size overflow
    (dict(scale=float("nan")), fa.FA_ERR_INVALID),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID),
    (dict(dt=7), fa.FA_ERR_INVALID),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=8), fa.FA_ERR_UNSUPPORTED),
    (dict(dt=fa.FA_F32, d=16), fa.FA_ERR_UNSUPPORTED),
    (dict(dt=fa.FA_F32, d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(N=(1 << 30) + 128), fa.FA_ERR_UNSUPPORTED),  # beyond the longest supported sequence
])
def test_fwd_rejects(lib, kwargs, status):
    assert fwd(lib, **kwargs) == status
    assert lib.fa_last_error().decode()


@pytest.mark.parametrize("kwargs, status", [
    (dict(mask=None), fa.FA_ERR_INVALID),
    (dict(mb=0), fa.FA_ERR_INVALID),
    (dict(mb=100), fa.FA_ERR_INVALID),
    (dict(mb=64), fa.FA_ERR_INVALID),
    (dict(N=4096 * 64 + 1), fa.FA_ERR_UNSUPPORTED),  # key-tile list capacity
])
def test_fwd_blocksparse_rejects(lib, kwargs, status):
    assert fwd_sparse(lib, **kwargs) == status


@pytest.mark.parametrize("kwargs, status", [
    (dict(dt=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_INVALID),
    (dict(ws=P + 16), fa.FA_ERR_INVALID),
    (dict(ws_bytes=100), fa.FA_ERR_INVALID),     # D for N=128 needs 512 bytes
    (dict(dq=0), fa.FA_ERR_INVALID),
    (dict(mask=P, mb=96), fa.FA_ERR_INVALID),
    (dict(mask=P, N=131072 + 1), fa.FA_ERR_UNSUPPORTED),  # query-tile list capacity (32-row steps)
    (dict(scale=float("nan")), fa.FA_ERR_INVALID),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
])
def test_bwd_rejects(lib, kwargs, status):
    assert bwd(lib, **kwargs) == status


def test_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        fa.fa_fwd(x, x, x, 0.125)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_LIB", None)
    monkeypatch.setattr(fa, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        fa.load()


def _kvcache_slots(B, H, Nk):
    # partial-result slots: at most 2048 waves (never more than the 32-key tiles of a full
    # cache) share the tiles of all (b, h); each wave leaves one partial per (b, h) it
    # touches, and slot w + bh is distinct for every such pair, so G + B H - 1 slots suffice
    tiles = B * H * -(-Nk // 32)
    return min(2048, max(tiles, 1)) + B * H - 1


@pytest.mark.parametrize("B,H,Nq,Nk,d", [(1, 1, 1, 1, 64), (8, 16, 1, 16384, 128), (4, 32, 16, 32768, 64),
                                         (2, 3, 5, 70000, 128), (1, 1, 32, 1 << 24, 64)])
def test_kvcache_workspace_bytes(lib, B, H, Nq, Nk, d):
    al = lambda x: (x + 255) // 256 * 256
    slots = _kvcache_slots(B, H, Nk)
    assert slots <= 2048 + B * H - 1
    rows = slots * Nq
    assert fa.fa_fwd_kvcache_workspace_bytes(B, H, Nq, Nk, d) == al(rows * d * 4) + 2 * al(rows * 4)
    assert fa.fa_fwd_kvcache_workspace_bytes(B, H, 0, Nk, d) == 0
    assert fa.fa_fwd_kvcache_workspace_bytes(B, H, Nq, -1, d) == 0


def kvc(lib, dt=fa.FA_BF16, B=1, H=1, Nq=1, Nk=256, d=64, q=P, k=P, v=P, o=P, lse=P, scale=0.125,
        kv_len=None, ws=P, ws_bytes=None):
    c = ctypes.c_void_p
    need = fa.fa_fwd_kvcache_workspace_bytes(B, H, Nq, Nk, d) if ws_bytes is None else ws_bytes
    return lib.fa_fwd_kvcache(dt, B, H, Nq, Nk, d, c(q), c(k), c(v), c(o), c(lse), scale, 1,
                              None if kv_len is None else c(kv_len), None if ws is None else c(ws), need, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(q=0), fa.FA_ERR_INVALID),
    (dict(k=P + 8), fa.FA_ERR_INVALID),
    (dict(lse=P + 2), fa.FA_ERR_INVALID),
    (dict(kv_len=P + 2), fa.FA_ERR_INVALID),
    (dict(Nq=0), fa.FA_ERR_INVALID),
    (dict(Nk=0), fa.FA_ERR_INVALID),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID),
    (dict(ws=None), fa.FA_ERR_INVALID),
    (dict(ws=P + 64), fa.FA_ERR_INVALID),
    (dict(ws_bytes=1000), fa.FA_ERR_INVALID),
    (dict(dt=7), fa.FA_ERR_INVALID),
    (dict(dt=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Nq=33), fa.FA_ERR_UNSUPPORTED),
    # 2^20 (b, h) x 2048 key tiles: the tile sequence would pass 2^31 - 1
    (dict(B=1024, H=1024, Nk=65536), fa.FA_ERR_UNSUPPORTED),
])
def test_kvcache_rejects(lib, kwargs, status):
    assert kvc(lib, **kwargs) == status
    assert lib.fa_last_error().decode()


def test_varlen_workspace_bytes(lib):
    al = lambda x: (x + 255) // 256 * 256
    for H, total, d in [(1, 1, 64), (12, 19432, 64), (16, 16384, 128), (2, 0, 64)]:
        assert fa.fa_bwd_varlen_workspace_bytes(H, total, d) == al(H * total * 4)
    assert fa.fa_bwd_varlen_workspace_bytes(0, 5, 64) == 0
    assert fa.fa_bwd_varlen_workspace_bytes(2, -1, 64) == 0


def fvar(lib, dt=fa.FA_BF16, nseq=2, H=2, total=300, max_seqlen=200, d=64, cu=P, q=P, o=P, lse=P,
         scale=0.125, causal=1, wl=-1, wr=-1):
    c = ctypes.c_void_p
    return lib.fa_fwd_varlen(dt, nseq, H, total, max_seqlen, d, None if cu is None else c(cu), c(q), c(P),
                             c(P), c(o), c(lse), scale, causal, wl, wr, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(cu=None), fa.FA_ERR_INVALID),
    (dict(cu=P + 2), fa.FA_ERR_INVALID),
    (dict(q=0), fa.FA_ERR_INVALID),
    (dict(o=P + 8), fa.FA_ERR_INVALID),
    (dict(lse=P + 1), fa.FA_ERR_INVALID),
    (dict(nseq=0), fa.FA_ERR_INVALID),
    (dict(H=0), fa.FA_ERR_INVALID),
    (dict(total=-1), fa.FA_ERR_INVALID),
    (dict(max_seqlen=-1), fa.FA_ERR_INVALID),
    (dict(max_seqlen=1 << 30, H=64, nseq=1 << 12), fa.FA_ERR_INVALID),  # grid size overflow
    (dict(wl=-2), fa.FA_ERR_INVALID),
    (dict(wr=-5), fa.FA_ERR_INVALID),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID),
    (dict(dt=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=48), fa.FA_ERR_UNSUPPORTED),
    (dict(max_seqlen=(1 << 30) + 1), fa.FA_ERR_UNSUPPORTED),
])
def test_varlen_rejects(lib, kwargs, status):
    assert fvar(lib, **kwargs) == status
    assert lib.fa_last_error().decode()


def test_varlen_no_tokens_launches_nothing(lib):
    # zero tokens: valid, returns before touching any tensor pointer (even NULL ones)
    assert fvar(lib, total=0, max_seqlen=0, q=0, o=0, lse=0) == fa.FA_OK


def test_varlen_bwd_rejects(lib):
    c = ctypes.c_void_p
    need = fa.fa_bwd_varlen_workspace_bytes(2, 300, 64)
    call = lambda ws, nbytes, dq=P: lib.fa_bwd_varlen(fa.FA_BF16, 2, 2, 300, 200, 64, c(P), c(P), c(P), c(P), c(P),
                                                      c(P), c(P), c(dq), c(P), c(P), 0.125, 1, -1, -1,
                                                      None if ws is None else c(ws), nbytes, None)
    assert call(None, need) == fa.FA_ERR_INVALID
    assert call(P + 16, need) == fa.FA_ERR_INVALID
    assert call(P, need - 1) == fa.FA_ERR_INVALID
    assert call(P, need, dq=0) == fa.FA_ERR_INVALID


def fdrop(lib, dt=fa.FA_BF16, p=0.1, seed=1, q=P):
    c = ctypes.c_void_p
    return lib.fa_fwd_dropout(dt, 1, 1, 128, 64, c(q), c(P), c(P), c(P), c(P), 0.125, 1, None, p, seed, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(p=-0.1), fa.FA_ERR_INVALID),
    (dict(p=1.0), fa.FA_ERR_INVALID),
    (dict(p=float("nan")), fa.FA_ERR_INVALID),
    (dict(dt=fa.FA_F32), fa.FA_ERR_UNSUPPORTED),
    (dict(q=0), fa.FA_ERR_INVALID),
])
def test_dropout_rejects(lib, kwargs, status):
    assert fdrop(lib, **kwargs) == status
    assert lib.fa_last_error().decode()


def test_dropout_bwd_rejects(lib):
    c = ctypes.c_void_p
    need = fa.fa_bwd_workspace_bytes(1, 1, 128, 64)
    call = lambda p, ws: lib.fa_bwd_dropout(fa.FA_BF16, 1, 1, 128, 64, c(P), c(P), c(P), c(P), c(P), c(P), c(P),
                                            c(P), c(P), 0.125, 1, None, p, 5, None if ws is None else c(ws), need,
                                            None)
    assert call(1.5, P) == fa.FA_ERR_INVALID
    assert call(0.2, None) == fa.FA_ERR_INVALID


def kvc_noalloc(lib, dt=fa.FA_BF16, B=1, H=1, Nq=1, Nk=256, d=64, q=P, o=P, lse=P, scale=0.125):
    c = ctypes.c_void_p
    return lib.fa_fwd_kvcache_noalloc(dt, B, H, Nq, Nk, d, c(q), c(P), c(P), c(o), c(lse), scale, 1, None, None)


@pytest.mark.parametrize("kwargs, status", [
    (dict(q=0), fa.FA_ERR_INVALID),
    (dict(lse=P + 2), fa.FA_ERR_INVALID),
    (dict(Nq=0), fa.FA_ERR_INVALID),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Nq=33), fa.FA_ERR_UNSUPPORTED),
    # partial results beyond the static scratch (102 MB: 2048 + 4095 slots x 32 queries x d=128)
    (dict(B=64, H=64, Nq=32, Nk=32, d=128), fa.FA_ERR_UNSUPPORTED),
])
def test_kvcache_noalloc_rejects(lib, kwargs, status):
    assert kvc_noalloc(lib, **kwargs) == status
    assert lib.fa_last_error().decode()


def test_last_error_is_per_thread(lib):
    """fa_last_error keeps each thread's own reason: two threads that fail validation in
    different ways, interleaved, always read back their own message (validation only; no
    device is touched)."""
    import threading
    results = {}
    barrier = threading.Barrier(2)

    def worker(name, kwargs, pattern):
        barrier.wait()
        ok = True
        for _ in range(300):
            st = fwd(lib, **kwargs)
            msg = lib.fa_last_error().decode()
            ok &= st != fa.FA_OK and re.search(pattern, msg) is not None
        results[name] = ok

    t1 = threading.Thread(target=worker, args=("sizes", dict(B=0), r"sizes must be positive"))
    t2 = threading.Thread(target=worker, args=("headdim", dict(d=96), r"head dimension 96"))
    t1.start()
    t2.start()
    t1.join()
    t2.join()
    assert results == {"sizes": True, "headdim": True}
