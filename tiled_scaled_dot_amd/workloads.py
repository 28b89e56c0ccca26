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

@dataclass(frozen=True)
class ScaledWorkload(Workload):
    """A workload of attn_fwd_scaled: base-2 weights with per-block scales
    (Q_scale per q_block query rows, K_scale per k_block keys); Q and K in
    ``qk_dtype`` (fp8_e4m3 or the 16-bit dtype), V and O in ``dtype``.
    Inputs come from ``scaled_inputs`` (the fp8 case quantises N(0,1) draws
    per block)."""
    q_block: int = 128
    k_block: int = 64
    qk_dtype: str = "fp8_e4m3"
    entry: str = "scaled"

    def min_bytes(self) -> int:
        qkb = 1 if self.qk_dtype == "fp8_e4m3" else DTYPES[self.qk_dtype].itemsize
        elt = DTYPES[self.dtype].itemsize
        nq, nk = -(-self.S_q // self.q_block), -(-self.S_k // self.k_block)
        per = (qkb * (self.S_q + self.S_k) * self.D_qk + elt * (self.S_k + self.S_q) * self.D_v
               + 4 * self.S_q + 4 * (nq + nk))
        return self.B * self.H * per


def _s(name, qk_dtype, causal, seed):
    return ScaledWorkload(name, "bf16", 1, 32, 16384, 16384, 128, 128, causal,
                          1.0 / math.sqrt(128), "normal", 1.0, 1.0, seed, q_block=128,
                          k_block=64, qk_dtype=qk_dtype)


# The long causal and non-causal cases with per-block scales: fp8 Q/K (the
# scores on the fp8 MFMA) and bf16 Q/K (the same chain at the 16-bit rate).
SCALED_WORKLOADS = {
    w.name: w for w in [
        _s("fp8qk_b1h32_s16384_d128_causal_scaled", "fp8_e4m3", True, 10),
        _s("fp8qk_b1h32_s16384_d128_scaled", "fp8_e4m3", False, 10),
        _s("bf16_b1h32_s16384_d128_causal_scaled", "bf16", True, 10),
    ]
}

ALL_WORKLOADS = {**WORKLOADS, **EXT_WORKLOADS, **SCALED_WORKLOADS}


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


def scaled_inputs(B, H, S_q, S_k, D_qk, D_v, q_block, k_block, qk_dtype: str, v_dtype: str,
                  seed: int, sigma: float = 1.0, sm_scale=None, scale_jitter: bool = False):
    """Inputs of the per-block scaled attention (seeded).

    Draws Q, K, V like ``random_inputs`` (normal, Q and K with std
    ``sigma``).  For ``qk_dtype == "fp8_e4m3"`` each block of q_block query
    rows (k_block keys) is divided by its absolute maximum / 448 and rounded
    to float8_e4m3fn; that factor times ``sm_scale * log2(e)`` (default
    sm_scale 1/sqrt(D_qk)) is the block's Q scale, the factor alone its K
    scale: the caller's quantisation step, which the method takes as given.
    For a 16-bit ``qk_dtype`` Q and K are rounded to it and the scales are
    ``sm_scale * log2(e)`` and 1, each times a factor drawn from [0.5, 1.5)
    per block when ``scale_jitter``.  Returns (q, k, v, q_scale, k_scale) on
    the CPU; the scales are float32 [B,H,blocks]."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    q = torch.randn((B, H, S_q, D_qk), generator=g) * sigma
    k = torch.randn((B, H, S_k, D_qk), generator=g) * sigma
    v = torch.randn((B, H, S_k, D_v), generator=g)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D_qk)
    c = sm_scale * 1.4426950408889634
    nq, nk = -(-S_q // q_block), -(-S_k // k_block)

    def per_block(x, blk, n):
        pad = n * blk - x.shape[2]
        xp = torch.nn.functional.pad(x, (0, 0, 0, pad))
        amax = xp.abs().reshape(B, H, n, blk * x.shape[3]).amax(-1)
        return torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))

    if qk_dtype == "fp8_e4m3":
        fq, fk = per_block(q, q_block, nq), per_block(k, k_block, nk)
        q8 = (q / fq.repeat_interleave(q_block, dim=2)[:, :, :S_q, None]).to(torch.float8_e4m3fn)
        k8 = (k / fk.repeat_interleave(k_block, dim=2)[:, :, :S_k, None]).to(torch.float8_e4m3fn)
        q_scale, k_scale = (fq * c).float(), fk.float()
        q, k = q8, k8
    else:
        q, k = q.to(DTYPES[qk_dtype]), k.to(DTYPES[qk_dtype])
        q_scale = torch.full((B, H, nq), c)
        k_scale = torch.ones((B, H, nk))
        if scale_jitter:
            q_scale = q_scale * (0.5 + torch.rand((B, H, nq), generator=g))
            k_scale = k_scale * (0.5 + torch.rand((B, H, nk), generator=g))
    return q, k, v.to(DTYPES[v_dtype]), q_scale.float().contiguous(), k_scale.float().contiguous()


def sample_rows(S_q: int, block_m: int = 128, stride: int = 17):
    """Query rows checked at full size: every `stride`-th row, rows 0, 1,
    S_q-1, and the rows on both sides of every `block_m` boundary.

    The default stride, 17, is coprime with 32, the query rows one wave of
    the kernels owns: over any 32 * 17 consecutive rows the stride-17 rows
    take every position 0..31 within their wave, so a fault tied to one lane
    position is not skipped."""
    rows = set(range(0, S_q, stride))
    rows.update({0, 1, S_q - 1})
    for b in range(block_m, S_q, block_m):
        rows.update({b - 1, b})
    return sorted(r for r in rows if 0 <= r < S_q)
