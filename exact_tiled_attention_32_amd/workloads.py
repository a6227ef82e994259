"""Seeded synthetic inputs for exact attention.

This module is the one piece shared by the HIP path's callers (tests, bench)
and the oracle's callers: it draws the inputs and holds none of the method's
arithmetic. All values are iid N(0, 1) from ``torch.Generator('cpu')``, drawn
in fp32 and rounded to bf16 (round-to-nearest-even) for the bf16 workloads, so
the GPU and the oracle consume the same bits.

The workloads stand in, by shape only, for the pages' benchmarks (BERT-large
at sequence length 512, GPT-2 at 1K, Long Range Arena at 16K and 64K); no
dataset or trained weight is involved.

Generation order per workload: Q, K, V, dO, then the key-padding lengths. Decode
workloads (a few queries against a key/value cache): Q [B, H, Nq, d], then the cache's
K and V [B, H, Nk, d], then the cache lengths. Packed variable-length workloads: the
sequence lengths first (when drawn), then Q, K, V, dO as [total, H, d].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "WORKLOADS", "generate", "sparse_block_rule", "make_case",
           "DecodeWorkload", "DECODE_WORKLOADS", "generate_decode", "make_decode_case",
           "VarlenWorkload", "VARLEN_WORKLOADS", "generate_varlen", "make_varlen_case"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "f32" or "bf16"
    seed: int
    causal: bool = False
    padding: bool = False  # key-padding lengths L_b ~ U{N/2 .. N} inclusive
    sparse: bool = False   # block mask from ``sparse_block_rule``
    mask_block: int = 128
    backward: bool = True
    description: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    "single_head_f32": Workload(
        "single_head_f32", 1, 1, 128, 64, "f32", 1001, backward=False,
        description="single-head forward, fp32, B=1 H=1 N=128 d=64, no mask"),
    "bert_padded": Workload(
        "bert_padded", 8, 16, 512, 64, "bf16", 1002, padding=True,
        description="BERT-large-shaped self-attention, bf16 fwd+bwd, B=8 H=16 N=512 d=64, "
                    "key padding with L_b uniform in [256, 512]"),
    "gpt2_causal": Workload(
        "gpt2_causal", 8, 12, 1024, 64, "bf16", 1003, causal=True,
        description="GPT-2-shaped causal attention, bf16 fwd+bwd, B=8 H=12 N=1024 d=64"),
    "long_causal_d64": Workload(
        "long_causal_d64", 1, 16, 16384, 64, "bf16", 1004, causal=True,
        description="long-sequence causal attention, bf16 fwd+bwd, B=1 H=16 N=16384 d=64"),
    "long_causal_d128": Workload(
        "long_causal_d128", 1, 16, 16384, 128, "bf16", 1014, causal=True,
        description="long-sequence causal attention, bf16 fwd+bwd, B=1 H=16 N=16384 d=128"),
    "long_causal_d32": Workload(
        "long_causal_d32", 1, 16, 16384, 32, "bf16", 1024, causal=True,
        description="long-sequence causal attention at the smallest built head dimension, bf16 "
                    "fwd+bwd, B=1 H=16 N=16384 d=32"),
    "long_causal_d16": Workload(
        "long_causal_d16", 1, 16, 16384, 16, "bf16", 1025, causal=True,
        description="long-sequence causal attention at head dimension 16 (32-wide tiles, upper "
                    "half zero), bf16 fwd+bwd, B=1 H=16 N=16384 d=16"),
    "block_sparse_64k": Workload(
        "block_sparse_64k", 1, 8, 65536, 64, "bf16", 1005, sparse=True,
        description="block-sparse attention, bf16 fwd+bwd, B=1 H=8 N=65536 d=64, 128x128 blocks, "
                    "block (i,j) kept iff |i-j| <= 1 or j mod 16 == 0"),
}


def sparse_block_rule(n_blocks: int) -> torch.Tensor:
    """uint8 [n_blocks, n_blocks]: 1 where |i - j| <= 1 or j % 16 == 0."""
    i = torch.arange(n_blocks).view(-1, 1)
    j = torch.arange(n_blocks).view(1, -1)
    return (((i - j).abs() <= 1) | (j % 16 == 0)).to(torch.uint8)


def _draw(gen, shape, dtype):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    return x if dtype == "f32" else x.to(torch.bfloat16)


def generate(w: Workload, *, with_grad_out: bool | None = None) -> dict:
    """CPU tensors for a workload: q, k, v, (do), kv_len (int32 or None), block_mask (uint8 or None)."""
    gen = torch.Generator("cpu").manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.d)
    q = _draw(gen, shape, w.dtype)
    k = _draw(gen, shape, w.dtype)
    v = _draw(gen, shape, w.dtype)
    need_do = w.backward if with_grad_out is None else with_grad_out
    do = _draw(gen, shape, w.dtype) if need_do else None
    kv_len = None
    if w.padding:
        kv_len = torch.randint(w.N // 2, w.N + 1, (w.B,), generator=gen, dtype=torch.int64).to(torch.int32)
    block_mask = None
    if w.sparse:
        block_mask = sparse_block_rule(-(-w.N // w.mask_block))
    return {"q": q, "k": k, "v": v, "do": do, "kv_len": kv_len, "block_mask": block_mask,
            "scale": w.scale, "causal": w.causal, "mask_block": w.mask_block}


def make_case(B: int, H: int, N: int, d: int, *, dtype: str = "bf16", seed: int = 0,
              causal: bool = False, kv_len=None, block_mask=None, mask_block: int = 128,
              q_magnitude: float = 1.0) -> dict:
    """A small seeded case for the parity sweep. ``kv_len`` may be a list of ints.

    ``q_magnitude`` multiplies Q before rounding: large values give scores with a
    standard deviation of about ``q_magnitude`` (scale = 1/sqrt(d)).
    """
    gen = torch.Generator("cpu").manual_seed(seed)
    shape = (B, H, N, d)

    def draw(mult=1.0):
        x = torch.randn(shape, generator=gen, dtype=torch.float32) * mult
        return x if dtype == "f32" else x.to(torch.bfloat16)

    q, k, v, do = draw(q_magnitude), draw(), draw(), draw()
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32)
    bm = None if block_mask is None else torch.as_tensor(block_mask, dtype=torch.uint8)
    return {"q": q, "k": k, "v": v, "do": do, "kv_len": kl, "block_mask": bm,
            "scale": 1.0 / math.sqrt(d), "causal": causal, "mask_block": mask_block}


@dataclass(frozen=True)
class DecodeWorkload:
    """Nq new queries per (b, h) against a cache of Nk keys and values."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    seed: int
    causal: bool = False
    padding: bool = False  # cache lengths L_b ~ U{Nk/2 .. Nk} inclusive
    description: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


DECODE_WORKLOADS = {
    "decode_q1_d128": DecodeWorkload(
        "decode_q1_d128", 8, 16, 1, 16384, 128, 1101, padding=True,
        description="single-query decode, bf16, B=8 H=16 Nq=1 against a 16K-entry cache, "
                    "d=128, cache lengths uniform in [8192, 16384]"),
    "decode_q16_causal_d64": DecodeWorkload(
        "decode_q16_causal_d64", 4, 32, 16, 32768, 64, 1102, causal=True, padding=True,
        description="16 new queries per head (causal among themselves), bf16, B=4 H=32 "
                    "against a 32K-entry cache, d=64, cache lengths uniform in [16384, 32768]"),
}


def generate_decode(w: DecodeWorkload) -> dict:
    """CPU bf16 tensors q [B,H,Nq,d], k, v [B,H,Nk,d] and kv_len (int32 or None)."""
    gen = torch.Generator("cpu").manual_seed(w.seed)
    q = _draw(gen, (w.B, w.H, w.Nq, w.d), "bf16")
    k = _draw(gen, (w.B, w.H, w.Nk, w.d), "bf16")
    v = _draw(gen, (w.B, w.H, w.Nk, w.d), "bf16")
    kv_len = None
    if w.padding:
        kv_len = torch.randint(w.Nk // 2, w.Nk + 1, (w.B,), generator=gen, dtype=torch.int64).to(torch.int32)
    return {"q": q, "k": k, "v": v, "kv_len": kv_len, "scale": w.scale, "causal": w.causal}


def make_decode_case(B: int, H: int, Nq: int, Nk: int, d: int, *, seed: int = 0, causal: bool = False,
                     kv_len=None, q_magnitude: float = 1.0) -> dict:
    """A small seeded bf16 decode case; ``kv_len`` may be a list of ints."""
    gen = torch.Generator("cpu").manual_seed(seed)
    q = (torch.randn((B, H, Nq, d), generator=gen) * q_magnitude).to(torch.bfloat16)
    k = torch.randn((B, H, Nk, d), generator=gen).to(torch.bfloat16)
    v = torch.randn((B, H, Nk, d), generator=gen).to(torch.bfloat16)
    kl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32)
    return {"q": q, "k": k, "v": v, "kv_len": kl, "scale": 1.0 / math.sqrt(d), "causal": causal}


@dataclass(frozen=True)
class VarlenWorkload:
    """Sequences packed along one token axis ([total, H, d]), optional sliding window."""
    name: str
    H: int
    d: int
    seed: int
    lengths: tuple = ()       # fixed lengths, or () to draw n_seq lengths U{lo .. hi}
    n_seq: int = 0
    lo: int = 0
    hi: int = 0
    causal: bool = False
    window_left: int = -1
    window_right: int = -1
    description: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


VARLEN_WORKLOADS = {
    "varlen_packed_causal": VarlenWorkload(
        "varlen_packed_causal", 12, 64, 1201, n_seq=16, lo=128, hi=2048, causal=True,
        description="16 causal sequences of lengths uniform in [128, 2048] packed into one "
                    "token axis, GPT-2-shaped heads (H=12, d=64), bf16 fwd+bwd"),
    "sliding_window_16k": VarlenWorkload(
        "sliding_window_16k", 16, 128, 1202, lengths=(16384,), causal=True, window_left=4095,
        description="one causal sequence of 16384 tokens with a 4096-key sliding window "
                    "(each query sees itself and the 4095 keys before it), H=16, d=128, bf16 fwd+bwd"),
}


def _varlen_tensors(gen, lengths, H, d, q_magnitude=1.0):
    total = int(sum(lengths))
    q = (torch.randn((total, H, d), generator=gen) * q_magnitude).to(torch.bfloat16)
    k, v, do = (torch.randn((total, H, d), generator=gen).to(torch.bfloat16) for _ in range(3))
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return q, k, v, do, cu


def generate_varlen(w: VarlenWorkload) -> dict:
    """CPU tensors q, k, v, do [total, H, d] (bf16), cu_seqlens (int32 [nseq + 1]) and the
    scalar arguments of a packed workload."""
    gen = torch.Generator("cpu").manual_seed(w.seed)
    if w.lengths:
        lengths = [int(x) for x in w.lengths]
    else:
        lengths = torch.randint(w.lo, w.hi + 1, (w.n_seq,), generator=gen, dtype=torch.int64).tolist()
    q, k, v, do, cu = _varlen_tensors(gen, lengths, w.H, w.d)
    return {"q": q, "k": k, "v": v, "do": do, "cu_seqlens": cu, "max_seqlen": max(lengths),
            "scale": w.scale, "causal": w.causal, "window_left": w.window_left,
            "window_right": w.window_right}


def make_varlen_case(lengths, H: int, d: int, *, seed: int = 0, causal: bool = False,
                     window_left: int = -1, window_right: int = -1, q_magnitude: float = 1.0) -> dict:
    """A small seeded packed case with the given sequence lengths."""
    gen = torch.Generator("cpu").manual_seed(seed)
    q, k, v, do, cu = _varlen_tensors(gen, list(lengths), H, d, q_magnitude)
    return {"q": q, "k": k, "v": v, "do": do, "cu_seqlens": cu, "max_seqlen": max(list(lengths) + [0]),
            "scale": 1.0 / math.sqrt(d), "causal": causal, "window_left": window_left,
            "window_right": window_right}
