"""fp64 CPU oracle for the attention forward pass — TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never links or calls
it, and it imports nothing from the GPU library.

``attn_ref`` evaluates the plain, non-online reference ``softmax(Q K^T *
scale) V`` per (batch, head) slice, plus the natural-log LSE, in double
precision (VeriTile, "FlashAttention1.NaiveRefinement", section "Naive FA
reference"; reduction order from tiny.accy.kernel.library.attention,
``expectedOutput``).  The arithmetic lives in ``attn_ref.c``; this module only
builds it with gcc and marshals numpy arrays through ctypes.

Every function here is pinned by ``tests/test_oracle.py`` (library routine,
high-precision brute force, closed forms, invariants, and planted mistakes).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attn_ref.c")
LIBRARY = os.path.join(_HERE, "liboracle_attn.so")

_lib = None


def build(force: bool = True, source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (no fast-math: IEEE double semantics);
    without ``force`` only when the library is missing or older than the
    source."""
    if (force or not os.path.exists(output)
            or os.path.getmtime(source) > os.path.getmtime(output)):
        tmp = output + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
               "-fno-fast-math", "-ffp-contract=off", source, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, output)
    return output


def load_library(path: str) -> ctypes.CDLL:
    lib = ctypes.CDLL(path)
    f = lib.attn_ref_f64
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    f.argtypes = [dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, i64, i64,
                  ctypes.c_double, ctypes.c_int, ctypes.POINTER(i64), i64,
                  ctypes.c_int]
    f.restype = ctypes.c_int
    g = lib.attn_ref_ext_f64
    g.argtypes = [dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, i64, i64, i64,
                  ctypes.c_double, ctypes.c_int, i64, i64, i64, i64,
                  ctypes.POINTER(i64), i64, ctypes.c_int]
    g.restype = ctypes.c_int
    h = lib.attn_ref_scaled_f64
    h.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, i64, i64, i64, i64,
                  ctypes.c_int, ctypes.POINTER(i64), i64, ctypes.c_int]
    h.restype = ctypes.c_int
    return lib


def _library() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build(force=False)
        _lib = load_library(LIBRARY)
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def attn_ref(q, k, v, scale: float, causal: bool, rows=None, nthreads=None,
             want_probs: bool = False, lib: ctypes.CDLL | None = None):
    """Return ``(O, LSE)`` (and the softmax weights ``P`` if asked).

    q: [B,H,S_q,D_qk], k: [B,H,S_k,D_qk], v: [B,H,S_k,D_v]; any float dtype,
    converted exactly to float64.  ``rows`` restricts the computation to the
    listed query rows (O then has shape [B,H,len(rows),D_v]).
    """
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B,H,S,D]")
    B, H, S_q, D_qk = q.shape
    if k.shape[:2] != (B, H) or v.shape[:2] != (B, H) or k.shape[3] != D_qk \
            or v.shape[2] != k.shape[2]:
        raise ValueError("inconsistent q/k/v shapes")
    S_k, D_v = k.shape[2], v.shape[3]
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows.shape[0]
        rows_p = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    else:
        n_rows, rows_p = S_q, None
    o = np.empty((B, H, n_rows, D_v), dtype=np.float64)
    lse = np.empty((B, H, n_rows), dtype=np.float64)
    p = np.empty((B, H, n_rows, S_k), dtype=np.float64) if want_probs else None
    lib = lib or _library()
    rc = lib.attn_ref_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(p),
                          B, H, S_q, S_k, D_qk, D_v, float(scale), int(bool(causal)),
                          rows_p, n_rows, int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"attn_ref_f64 failed with status {rc}")
    return (o, lse, p) if want_probs else (o, lse)


def attn_ref_ext(q, k, v, scale: float, causal: bool, causal_offset: int = 0,
                 window: int = 0, kv_begin: int = 0, kv_end=None, rows=None,
                 nthreads=None, want_probs: bool = False, lib: ctypes.CDLL | None = None):
    """``attn_ref`` with each query row i restricted to the keys j with
    kv_begin <= j < kv_end, j <= i + causal_offset (causal) and
    j > i + causal_offset - window (window > 0).  Rows without a visible
    key give O = 0 and LSE = -inf.  k and v may hold fewer heads than q
    (H_kv dividing H): query head h then reads K/V head h // (H // H_kv)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B,H,S,D]")
    B, H, S_q, D_qk = q.shape
    H_kv = k.shape[1]
    if k.shape[0] != B or v.shape[:2] != (B, H_kv) or k.shape[3] != D_qk \
            or v.shape[2] != k.shape[2] or H_kv < 1 or H % H_kv != 0:
        raise ValueError("inconsistent q/k/v shapes")
    S_k, D_v = k.shape[2], v.shape[3]
    if kv_end is None:
        kv_end = S_k
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows.shape[0]
        rows_p = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    else:
        n_rows, rows_p = S_q, None
    o = np.empty((B, H, n_rows, D_v), dtype=np.float64)
    lse = np.empty((B, H, n_rows), dtype=np.float64)
    p = np.empty((B, H, n_rows, S_k), dtype=np.float64) if want_probs else None
    lib = lib or _library()
    rc = lib.attn_ref_ext_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(p),
                              B, H, H_kv, S_q, S_k, D_qk, D_v, float(scale),
                              int(bool(causal)),
                              int(causal_offset), int(window), int(kv_begin), int(kv_end),
                              rows_p, n_rows, int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"attn_ref_ext_f64 failed with status {rc}")
    return (o, lse, p) if want_probs else (o, lse)


def attn_ref_scaled(q, k, v, q_scale, k_scale, q_block: int, k_block: int, causal: bool,
                    rows=None, nthreads=None, want_probs: bool = False,
                    lib: ctypes.CDLL | None = None):
    """Base-2 attention with per-block scales: s_ij = q_scale[b,h,i//q_block]
    * k_scale[b,h,j//k_block] * (q_i . k_j), weights 2^s_ij normalised per
    row, LSE = ln sum_j 2^s_ij (natural log).  q_scale [B,H,ceil(S_q/q_block)],
    k_scale [B,H,ceil(S_k/k_block)]; causal is top-left."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    qs = np.ascontiguousarray(q_scale, dtype=np.float64)
    ks = np.ascontiguousarray(k_scale, dtype=np.float64)
    B, H, S_q, D_qk = q.shape
    S_k, D_v = k.shape[2], v.shape[3]
    if k.shape != (B, H, S_k, D_qk) or v.shape[:3] != (B, H, S_k):
        raise ValueError("inconsistent q/k/v shapes")
    if qs.shape != (B, H, -(-S_q // q_block)) or ks.shape != (B, H, -(-S_k // k_block)):
        raise ValueError("scale arrays do not match the block sizes")
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows.shape[0]
        rows_p = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    else:
        n_rows, rows_p = S_q, None
    o = np.empty((B, H, n_rows, D_v), dtype=np.float64)
    lse = np.empty((B, H, n_rows), dtype=np.float64)
    p = np.empty((B, H, n_rows, S_k), dtype=np.float64) if want_probs else None
    lib = lib or _library()
    rc = lib.attn_ref_scaled_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(p),
                                 _ptr(qs), _ptr(ks), B, H, S_q, S_k, D_qk, D_v, int(q_block),
                                 int(k_block), int(bool(causal)), rows_p, n_rows,
                                 int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"attn_ref_scaled_f64 failed with status {rc}")
    return (o, lse, p) if want_probs else (o, lse)


def merge_ref(o_parts, lse_parts):
    """Combine partial results over disjoint key sets (fp64, plain formula):
    LSE = ln sum_g exp(LSE_g) and O = sum_g exp(LSE_g - LSE) O_g.  A part
    with LSE_g = -inf contributes nothing; if every part is empty the result
    is O = 0, LSE = -inf."""
    lse_parts = [np.asarray(x, dtype=np.float64) for x in lse_parts]
    o_parts = [np.asarray(x, dtype=np.float64) for x in o_parts]
    m = np.max(np.stack(lse_parts), axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    total = np.zeros_like(m_safe)
    for lg in lse_parts:
        total += np.where(np.isfinite(lg), np.exp(lg - m_safe), 0.0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, total, 1.0)), -np.inf)
    o = np.zeros_like(o_parts[0])
    for og, lg in zip(o_parts, lse_parts):
        wgt = np.where(np.isfinite(lg) & finite, np.exp(lg - np.where(finite, lse, 0.0)), 0.0)
        o += wgt[..., None] * og
    return o, lse
