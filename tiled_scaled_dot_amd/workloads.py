"""Seeded synthetic workloads for the attention forward pass.

This module holds the workload table and the seeded input generators that
both the GPU library's tests/benchmark and the CPU oracle consume.  It holds
none of the method's arithmetic: it only draws random numbers and rounds them
to the storage dtype.

Generation recipe (fixed so every consumer sees identical inputs):
``g = torch.Generator('cpu').manual_seed(seed)``; draw Q, then K, then V in
float32 with ``randn(shape) * sigma`` (normal) or ``2 * rand(shape) - 1``
(uniform on [-1, 1)); then ``.to(dtype)`` (round to nearest even).  The
oracle receives exactly those rounded values, widened to float64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    B: int
    H: int
    S_q: int
    S_k: int
    D_qk: int
    D_v: int
    causal: bool
    scale: float
    dist: str          # "normal" or "uniform"
    sigma_qk: float    # std of Q and K (normal only)
    sigma_v: float     # std of V (normal only)
    seed: int

    @property
    def shape_q(self):
        return (self.B, self.H, self.S_q, self.D_qk)

    @property
    def shape_k(self):
        return (self.B, self.H, self.S_k, self.D_qk)

    @property
    def shape_v(self):
        return (self.B, self.H, self.S_k, self.D_v)

    @property
    def shape_o(self):
        return (self.B, self.H, self.S_q, self.D_v)

    def metric_flops(self) -> float:
        """2*B*H*S_q*S_k*(D_qk+D_v), halved when causal (the headline count)."""
        f = 2.0 * self.B * self.H * self.S_q * self.S_k * (self.D_qk + self.D_v)
        return f / 2.0 if self.causal else f

    def exact_pairs(self) -> int:
        """Number of visible (query, key) pairs per slice."""
        if not self.causal:
            return self.S_q * self.S_k
        # query i sees min(i + 1, S_k) keys (top-left alignment)
        n = min(self.S_q, self.S_k)
        tri = n * (n + 1) // 2
        return tri + max(0, self.S_q - self.S_k) * self.S_k

    def min_bytes(self) -> int:
        """Q + K + V read once, O written once (storage dtype), LSE (f32)."""
        elt = DTYPES[self.dtype].itemsize
        per = elt * (self.S_q * self.D_qk + self.S_k * self.D_qk
                     + self.S_k * self.D_v + self.S_q * self.D_v) + 4 * self.S_q
        return self.B * self.H * per

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _w(name, dtype, B, H, S_q, S_k, D_qk, D_v, causal, dist, sigma_qk, sigma_v,
       seed, scale=None):
    return Workload(name, dtype, B, H, S_q, S_k, D_qk, D_v, causal,
                    scale if scale is not None else 1.0 / math.sqrt(D_qk),
                    dist, sigma_qk, sigma_v, seed)


SQ3 = math.sqrt(3.0)

# The five workload families the target names, one entry per variant.
WORKLOADS = {
    "f32_b1h2_s128_d64": _w("f32_b1h2_s128_d64", "f32", 1, 2, 128, 128, 64, 64,
                            False, "normal", 1.0, 1.0, 1),
    "f32_b2h4_q1000_k777_d80": _w("f32_b2h4_q1000_k777_d80", "f32", 2, 4, 1000, 777,
                                  80, 80, False, "normal", 1.0, 1.0, 2),
    "f32_b2h4_q1000_k777_d80_causal": _w("f32_b2h4_q1000_k777_d80_causal", "f32", 2, 4,
                                         1000, 777, 80, 80, True, "normal", 1.0, 1.0, 2),
    "bf16_b4h16_s4096_d128_causal": _w("bf16_b4h16_s4096_d128_causal", "bf16", 4, 16,
                                       4096, 4096, 128, 128, True, "normal", 1.0, 1.0, 3),
    "bf16_b1h32_s16384_d128_causal": _w("bf16_b1h32_s16384_d128_causal", "bf16", 1, 32,
                                        16384, 16384, 128, 128, True, "normal", 1.0, 1.0, 4),
    "bf16_b1h32_s16384_d128_causal_var3": _w("bf16_b1h32_s16384_d128_causal_var3", "bf16",
                                             1, 32, 16384, 16384, 128, 128, True,
                                             "normal", SQ3, 1.0, 40),
    "bf16_b1h32_s16384_d128": _w("bf16_b1h32_s16384_d128", "bf16", 1, 32, 16384, 16384,
                                 128, 128, False, "normal", 1.0, 1.0, 4),
    "bf16_b1h32_s16384_d128_var3": _w("bf16_b1h32_s16384_d128_var3", "bf16", 1, 32,
                                      16384, 16384, 128, 128, False, "normal", SQ3, 1.0, 40),
    "f16_b4h16_q2048_k8192_dqk64_dv128": _w("f16_b4h16_q2048_k8192_dqk64_dv128", "f16",
                                            4, 16, 2048, 8192, 64, 128, False,
                                            "uniform", 1.0, 1.0, 5),
}

# The headline benchmark workload: bf16, causal, S = 16384, D = 128.
HEADLINE = "bf16_b1h32_s16384_d128_causal"


@dataclass(frozen=True)
class ExtWorkload(Workload):
    """A workload of the extended entry points: row i sees the keys
    [max(0, i + causal_offset - window + 1) if window else 0,
     min(S_k, i + causal_offset + 1) if causal else S_k).
    entry: "ext" (attn_fwd_ext, one launch) or "splitkv" (attn_fwd_partial
    over key chunks, then attn_merge; n_splits 0 = the library's choice).
    H_kv: K/V heads (0 = H); query head h reads K/V head h // (H // H_kv)."""
    causal_offset: int = 0
    window: int = 0
    entry: str = "ext"
    n_splits: int = 0
    H_kv: int = 0

    @property
    def kv_heads(self) -> int:
        return self.H_kv or self.H

    @property
    def shape_k(self):
        return (self.B, self.kv_heads, self.S_k, self.D_qk)

    @property
    def shape_v(self):
        return (self.B, self.kv_heads, self.S_k, self.D_v)

    def row_ranges(self):
        import numpy as np

        i = np.arange(self.S_q, dtype=np.int64)
        lo = np.zeros_like(i)
        if self.window > 0:
            lo = np.maximum(lo, i + self.causal_offset - self.window + 1)
        hi = np.full_like(i, self.S_k)
        if self.causal:
            hi = np.minimum(hi, i + self.causal_offset + 1)
        return lo, np.maximum(hi, lo)

    def visible_pairs(self) -> int:
        lo, hi = self.row_ranges()
        return int((hi - lo).sum())

    def metric_flops(self) -> float:
        """2 * (D_qk + D_v) per visible (query, key) pair."""
        return 2.0 * self.B * self.H * self.visible_pairs() * (self.D_qk + self.D_v)

    def key_span(self) -> int:
        lo, hi = self.row_ranges()
        live = hi > lo
        return int(hi[live].max() - lo[live].min()) if live.any() else 0

    def min_bytes(self) -> int:
        """Q, the keys and values some row sees (once per K/V head), O
        (storage dtype) and LSE."""
        elt = DTYPES[self.dtype].itemsize
        per_q = elt * (self.S_q * self.D_qk + self.S_q * self.D_v) + 4 * self.S_q
        per_kv = elt * self.key_span() * (self.D_qk + self.D_v)
        return self.B * (self.H * per_q + self.kv_heads * per_kv)


def _x(name, B, H, S_q, S_k, D, causal, causal_offset, window, entry, seed, n_splits=0,
       H_kv=0):
    return ExtWorkload(name, "bf16", B, H, S_q, S_k, D, D, causal, 1.0 / math.sqrt(D),
                       "normal", 1.0, 1.0, seed, causal_offset=causal_offset, window=window,
                       entry=entry, n_splits=n_splits, H_kv=H_kv)


# Workloads of the extended entry points (measured, not part of the target's
# table): a chunk of 512 new queries against a 128k-key context and one
# decoding query per sequence against 16k keys, both with the diagonal at
# the bottom right, each with and without key chunks; the decoding case
# again with 8 K/V heads for the 32 query heads; and the long causal case
# with a 4096-key sliding window.
EXT_WORKLOADS = {
    w.name: w for w in [
        _x("bf16_b1h8_q512_k131072_d128_prefill_splitkv", 1, 8, 512, 131072, 128, True,
           131072 - 512, 0, "splitkv", 6),
        _x("bf16_b1h8_q512_k131072_d128_prefill_nosplit", 1, 8, 512, 131072, 128, True,
           131072 - 512, 0, "ext", 6),
        _x("bf16_b4h32_q1_k16384_d128_decode_splitkv", 4, 32, 1, 16384, 128, True,
           16384 - 1, 0, "splitkv", 7),
        _x("bf16_b4h32_q1_k16384_d128_decode_nosplit", 4, 32, 1, 16384, 128, True,
           16384 - 1, 0, "ext", 7),
        _x("bf16_b4h32kv8_q1_k16384_d128_decode_splitkv", 4, 32, 1, 16384, 128, True,
           16384 - 1, 0, "splitkv", 9, H_kv=8),
        _x("bf16_b1h32_s16384_d128_causal_window4096", 1, 32, 16384, 16384, 128, True,
           0, 4096, "ext", 8),
    ]
}

ALL_WORKLOADS = {**WORKLOADS, **EXT_WORKLOADS}


def make_inputs(w: Workload, device="cpu"):
    """Return (q, k, v) in the workload's storage dtype (CPU unless asked)."""
    g = torch.Generator(device="cpu").manual_seed(w.seed)
    if w.dist == "normal":
        q = torch.randn(w.shape_q, generator=g) * w.sigma_qk
        k = torch.randn(w.shape_k, generator=g) * w.sigma_qk
        v = torch.randn(w.shape_v, generator=g) * w.sigma_v
    elif w.dist == "uniform":
        q = 2.0 * torch.rand(w.shape_q, generator=g) - 1.0
        k = 2.0 * torch.rand(w.shape_k, generator=g) - 1.0
        v = 2.0 * torch.rand(w.shape_v, generator=g) - 1.0
    else:
        raise ValueError(f"unknown distribution {w.dist!r}")
    dt = DTYPES[w.dtype]
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    if device != "cpu":
        q, k, v = q.to(device), k.to(device), v.to(device)
    return q, k, v


def random_inputs(shape_q, shape_k, shape_v, dtype: str, seed: int,
                  sigma: float = 1.0):
    """Normal inputs of arbitrary shape (for edge-case tests)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    dt = DTYPES[dtype]
    q = (torch.randn(shape_q, generator=g) * sigma).to(dt)
    k = (torch.randn(shape_k, generator=g) * sigma).to(dt)
    v = torch.randn(shape_v, generator=g).to(dt)
    return q, k, v


def sample_rows(S_q: int, block_m: int = 128, stride: int = 16):
    """Query rows checked at full size: every `stride`-th row, rows 0, 1,
    S_q-1, and the rows on both sides of every `block_m` boundary."""
    rows = set(range(0, S_q, stride))
    rows.update({0, 1, S_q - 1})
    for b in range(block_m, S_q, block_m):
        rows.update({b - 1, b})
    return sorted(r for r in rows if 0 <= r < S_q)
