"""Pins for the fp64 oracle: checks that tie it to something other than itself.

Each pin takes a loaded oracle library (the real one, or a copy with a
planted mistake) and raises AssertionError when the oracle disagrees with
what the pages and the mathematics fix:

* a library routine: torch's scaled_dot_product_attention (math path, fp64
  CPU) and torch.logsumexp, which compute the same definition;
* a high-precision brute force (mpmath, 40 digits) of the textbook softmax
  without the max shift, so a wrong or missing shift shows up;
* closed forms: one key, Q = 0 / scale = 0, the first causal query, two keys
  (logistic weights), a dominant key, scores far from zero;
* invariants: weights sum to one, key permutation, score shift, linearity in
  V, causal prefix, zero padding of the head dims, row sampling, threads;
* the worked example printed on tiny.accy.kernel.library.attention;
* for the extended entry point (key range, signed causal offset, window):
  torch's fp64 attention on the truncated key prefix, the 40-digit brute
  force on explicit key sets, a one-key window, rows without keys, and the
  merge of partial results over a key partition.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import mpmath
import numpy as np
import scipy.special
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _ref(lib, q, k, v, scale, causal, **kw):
    return oracle.attn_ref(q, k, v, scale, causal, lib=lib, nthreads=kw.pop("nthreads", 2), **kw)


def _randn(rng, *shape, sigma=1.0):
    return rng.standard_normal(shape) * sigma


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max rel err {err:.3e} > {tol:.1e}"


def _library_sdpa(q, k, v, scale, causal):
    Q, K, V = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal,
                                                         scale=scale)
    s = torch.matmul(Q, K.transpose(-1, -2).contiguous()) * scale
    if causal:
        mask = torch.ones(s.shape[-2], s.shape[-1], dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


# ---------------------------------------------------------------- library routine
LIB_CASES = [
    # B, H, S_q, S_k, D_qk, D_v, scale
    (1, 1, 1, 1, 1, 1, 0.5),
    (2, 3, 7, 5, 4, 6, 0.37),
    (1, 2, 5, 9, 3, 2, -0.8),
    (1, 1, 33, 17, 16, 8, 0.0),
    (2, 2, 64, 64, 32, 32, 1 / math.sqrt(32)),
    (1, 1, 13, 40, 5, 7, 2.5),
    (1, 2, 70, 45, 80, 80, 1 / math.sqrt(80)),
]


def pin_library_sdpa(lib):
    rng = np.random.default_rng(11)
    for (B, H, S_q, S_k, D_qk, D_v, scale), causal in itertools.product(LIB_CASES, (False, True)):
        q = _randn(rng, B, H, S_q, D_qk)
        k = _randn(rng, B, H, S_k, D_qk)
        v = _randn(rng, B, H, S_k, D_v)
        o, lse = _ref(lib, q, k, v, scale, causal)
        o_t, lse_t = _library_sdpa(q, k, v, scale, causal)
        tag = f"sdpa B{B}H{H} {S_q}x{S_k} d{D_qk}/{D_v} s{scale:.3f} c{causal}"
        _close(o, o_t, 1e-12, tag + " O")
        _close(lse, lse_t, 1e-12, tag + " LSE")


# ------------------------------------------------------- high-precision brute force
def _mp_attention_row(q, K, V, scale, n_valid):
    """Textbook softmax with no max shift, evaluated with 40 significant digits."""
    with mpmath.workdps(40):
        s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b))
                                             for a, b in zip(q, K[j])) for j in range(n_valid)]
        e = [mpmath.exp(x) for x in s]
        z = mpmath.fsum(e)
        out = [mpmath.fsum(e[j] * mpmath.mpf(float(V[j][c])) for j in range(n_valid)) / z
               for c in range(len(V[0]))]
        return [float(x) for x in out], float(mpmath.log(z))


def pin_highprec_unshifted(lib):
    rng = np.random.default_rng(12)
    for S_q, S_k, D_qk, D_v, causal in itertools.product((1, 2, 5), (1, 3, 6), (1, 3),
                                                           (1, 2), (False, True)):
        scale = float(rng.uniform(0.2, 1.5)) * (1 if rng.random() < 0.7 else -1)
        q = _randn(rng, 1, 1, S_q, D_qk, sigma=2.0)
        k = _randn(rng, 1, 1, S_k, D_qk, sigma=2.0)
        v = _randn(rng, 1, 1, S_k, D_v)
        o, lse = _ref(lib, q, k, v, scale, causal)
        for i in range(S_q):
            n_valid = min(i + 1, S_k) if causal else S_k
            o_mp, lse_mp = _mp_attention_row(q[0, 0, i], k[0, 0], v[0, 0], scale, n_valid)
            tag = f"mp {S_q}x{S_k} d{D_qk}/{D_v} c{causal} row{i}"
            _close(o[0, 0, i], o_mp, 1e-13, tag + " O")
            _close(lse[0, 0, i], lse_mp, 1e-13, tag + " LSE")


# ------------------------------------------------------------------- closed forms
def pin_single_key(lib):
    rng = np.random.default_rng(13)
    for causal in (False, True):
        q = _randn(rng, 2, 2, 6, 5)
        k = _randn(rng, 2, 2, 1, 5)
        v = _randn(rng, 2, 2, 1, 3)
        o, lse = _ref(lib, q, k, v, 0.7, causal)
        _close(o, np.broadcast_to(v, o.shape), 1e-15, "single key O = V[0]")
        s0 = 0.7 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0])
        _close(lse, s0, 1e-13, "single key LSE = s_0")


def pin_uniform_weights(lib):
    """Q = 0 or scale = 0: every score is 0, O is the mean of the visible V rows."""
    rng = np.random.default_rng(14)
    S_q, S_k = 9, 6
    for causal, zero_q in itertools.product((False, True), (False, True)):
        q = np.zeros((1, 2, S_q, 4)) if zero_q else _randn(rng, 1, 2, S_q, 4)
        scale = 0.9 if zero_q else 0.0
        k = _randn(rng, 1, 2, S_k, 4)
        v = _randn(rng, 1, 2, S_k, 3)
        o, lse = _ref(lib, q, k, v, scale, causal)
        for i in range(S_q):
            n = min(i + 1, S_k) if causal else S_k
            _close(o[:, :, i], v[:, :, :n].mean(axis=2), 1e-14, f"mean of V row {i}")
            _close(lse[:, :, i], np.full((1, 2), math.log(n)), 1e-14, f"ln|J| row {i}")


def pin_first_causal_query(lib):
    rng = np.random.default_rng(15)
    q = _randn(rng, 2, 3, 4, 6)
    k = _randn(rng, 2, 3, 7, 6)
    v = _randn(rng, 2, 3, 7, 5)
    o, lse = _ref(lib, q, k, v, 0.45, True)
    _close(o[:, :, 0], v[:, :, 0], 1e-15, "causal row 0 O = V[0]")
    _close(lse[:, :, 0], 0.45 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), 1e-13,
           "causal row 0 LSE")


def pin_two_keys(lib):
    rng = np.random.default_rng(16)
    q = _randn(rng, 1, 3, 5, 4, sigma=2.0)
    k = _randn(rng, 1, 3, 2, 4, sigma=2.0)
    v = _randn(rng, 1, 3, 2, 3)
    scale = 0.8
    o, lse = _ref(lib, q, k, v, scale, False)
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    w0 = scipy.special.expit(s[..., 0] - s[..., 1])[..., None]
    w1 = scipy.special.expit(s[..., 1] - s[..., 0])[..., None]
    expect = w0 * v[:, :, None, 0, :] + w1 * v[:, :, None, 1, :]
    _close(o, expect, 1e-13, "two keys O (logistic)")
    _close(lse, np.logaddexp(s[..., 0], s[..., 1]), 1e-13, "two keys LSE (logaddexp)")


def pin_far_scores(lib):
    """A dominant key takes all the weight; scores near +-2000 need the max shift."""
    # dominant key: scores 100 vs <= 40 -> other weights below e^-60
    q = np.zeros((1, 1, 1, 2))
    q[..., 0] = 1.0
    k = np.array([[[[100.0, 0.0], [40.0, 0.0], [-30.0, 1.0], [10.0, 5.0]]]])
    v = np.arange(8, dtype=np.float64).reshape(1, 1, 4, 2) + 1.0
    o, lse = _ref(lib, q, k, v, 1.0, False)
    _close(o[0, 0, 0], v[0, 0, 0], 1e-20, "dominant key")
    _close(lse[0, 0, 0], 100.0, 1e-15, "dominant key LSE")
    # all scores near +-2000: exp() of them overflows / underflows without a shift
    t = np.array([0.3, -1.1, 0.8, 0.0, 2.0])
    w = scipy.special.softmax(t)
    v = np.random.default_rng(17).standard_normal((1, 1, 5, 3))
    for base in (-2000.0, 2000.0):
        k = np.zeros((1, 1, 5, 2))
        k[0, 0, :, 0] = base + t
        o, lse = _ref(lib, q, k, v, 1.0, False)
        _close(o[0, 0, 0], w @ v[0, 0], 1e-12, f"scores near {base} O")
        _close(lse[0, 0, 0], base + scipy.special.logsumexp(t), 1e-15, f"scores near {base} LSE")


# --------------------------------------------------------------------- invariants
def pin_weights_sum_to_one(lib):
    rng = np.random.default_rng(18)
    for causal in (False, True):
        q = _randn(rng, 2, 2, 11, 7, sigma=2.0)
        k = _randn(rng, 2, 2, 8, 7, sigma=2.0)
        v = _randn(rng, 2, 2, 8, 3)
        o, lse, p = _ref(lib, q, k, v, 0.6, causal, want_probs=True)
        _close(p.sum(axis=-1), np.ones(p.shape[:-1]), 1e-14, "rows of P sum to 1")
        assert np.all(p >= 0.0)
        if causal:
            upper = np.triu(np.ones((11, 8), dtype=bool), k=1)
            assert np.all(p[..., upper] == 0.0), "causal: weight on a future key"
        _close(o, np.einsum("bhij,bhjc->bhic", p, v), 1e-13, "O = P V")


def pin_key_permutation(lib):
    rng = np.random.default_rng(19)
    q = _randn(rng, 1, 2, 6, 5)
    k = _randn(rng, 1, 2, 9, 5)
    v = _randn(rng, 1, 2, 9, 4)
    perm = rng.permutation(9)
    o1, l1 = _ref(lib, q, k, v, 0.5, False)
    o2, l2 = _ref(lib, q, k[:, :, perm], v[:, :, perm], 0.5, False)
    _close(o2, o1, 1e-14, "key permutation O")
    _close(l2, l1, 1e-14, "key permutation LSE")


def pin_score_shift(lib):
    rng = np.random.default_rng(20)
    for causal in (False, True):
        q = _randn(rng, 1, 2, 7, 5)
        k = _randn(rng, 1, 2, 6, 5)
        v = _randn(rng, 1, 2, 6, 4)
        u = _randn(rng, 5)
        o1, l1 = _ref(lib, q, k, v, 0.7, causal)
        o2, l2 = _ref(lib, q, k + u, v, 0.7, causal)
        _close(o2, o1, 1e-13, "score shift O")
        _close(l2, l1 + 0.7 * (q @ u), 1e-13, "score shift LSE")


def pin_linear_in_v(lib):
    rng = np.random.default_rng(21)
    for causal in (False, True):
        q = _randn(rng, 1, 1, 8, 4)
        k = _randn(rng, 1, 1, 5, 4)
        v = _randn(rng, 1, 1, 5, 3)
        a = _randn(rng, 3, 6)
        b = _randn(rng, 6)
        o1, _ = _ref(lib, q, k, v, 0.9, causal)
        o2, _ = _ref(lib, q, k, v @ a + b, 0.9, causal)
        _close(o2, o1 @ a + b, 1e-13, "O(VA + 1b^T) = O(V)A + 1b^T")


def pin_causal_prefix(lib):
    rng = np.random.default_rng(22)
    S_q, S_k = 10, 6
    q = _randn(rng, 1, 2, S_q, 4)
    k = _randn(rng, 1, 2, S_k, 4)
    v = _randn(rng, 1, 2, S_k, 3)
    oc, lc = _ref(lib, q, k, v, 0.8, True)
    for i in range(S_q):
        n = min(i + 1, S_k)
        on, ln = _ref(lib, q[:, :, i:i + 1], k[:, :, :n], v[:, :, :n], 0.8, False)
        _close(oc[:, :, i], on[:, :, 0], 1e-15, f"causal row {i} = prefix attention")
        _close(lc[:, :, i], ln[:, :, 0], 1e-15, f"causal LSE row {i}")


def pin_head_dim_padding(lib):
    rng = np.random.default_rng(23)
    q = _randn(rng, 1, 2, 5, 3)
    k = _randn(rng, 1, 2, 7, 3)
    v = _randn(rng, 1, 2, 7, 2)
    o1, l1 = _ref(lib, q, k, v, 0.6, True)
    qp = np.concatenate([q, np.zeros((1, 2, 5, 5))], axis=-1)
    kp = np.concatenate([k, np.zeros((1, 2, 7, 5))], axis=-1)
    vp = np.concatenate([v, _randn(rng, 1, 2, 7, 6)], axis=-1)
    o2, l2 = _ref(lib, qp, kp, vp, 0.6, True)
    assert np.array_equal(o2[..., :2], o1), "zero-padded head dims change O"
    assert np.array_equal(l2, l1), "zero-padded head dims change LSE"


def pin_rows_and_threads(lib):
    rng = np.random.default_rng(24)
    q = _randn(rng, 2, 3, 30, 6)
    k = _randn(rng, 2, 3, 21, 6)
    v = _randn(rng, 2, 3, 21, 5)
    rows = [0, 1, 7, 20, 21, 29]
    for causal in (False, True):
        o1, l1 = _ref(lib, q, k, v, 0.4, causal, nthreads=1)
        o4, l4 = _ref(lib, q, k, v, 0.4, causal, nthreads=5)
        assert np.array_equal(o1, o4) and np.array_equal(l1, l4), "thread count changes result"
        orow, lrow = _ref(lib, q, k, v, 0.4, causal, rows=rows, nthreads=3)
        assert np.array_equal(orow, o1[:, :, rows]), "row sampling changes O"
        assert np.array_equal(lrow, l1[:, :, rows]), "row sampling changes LSE"


# --------------------------------------------------------------- worked example
def load_page_example():
    with open(os.path.join(GOLDEN, "page3_worked_example.json")) as f:
        g = json.load(f)
    q = np.array(g["query"], dtype=np.float64)[:, None]
    k = np.array(g["key"], dtype=np.float64)[:, None]
    v = np.array(g["value"], dtype=np.float64)[:, None]
    return g, q, k, v


def _page_order_f32(q, k, v, scale):
    """A float32 evaluation of the chain the page's check follows, written
    with whole-array operations: the dot products, then the scale; the row
    max, seeded with -inf; the sum over keys of exp(score - max); each
    weight as that exp divided by the sum; the weighted sum of the value
    rows.  Only the rounding differs from the fp64 oracle, so the two agree
    to the page's float32 tolerance."""
    q32, k32, v32 = (np.asarray(x, dtype=np.float32) for x in (q, k, v))
    scores = np.matmul(q32, np.swapaxes(k32, -1, -2)).astype(np.float32) * np.float32(scale)
    row_max = np.max(scores, axis=-1, initial=np.float32(-np.inf), keepdims=True)
    shifted = np.exp((scores - row_max).astype(np.float32))
    denom = np.sum(shifted, axis=-1, keepdims=True, dtype=np.float32)
    weights = (shifted / denom).astype(np.float32)
    return np.matmul(weights, v32).astype(np.float32)


def pin_page_worked_example(lib):
    g, q, k, v = load_page_example()
    scale = 1.0 / math.sqrt(g["qk"])
    o, lse = _ref(lib, q, k, v, scale, False)
    o_t, lse_t = _library_sdpa(q, k, v, scale, False)
    _close(o, o_t, 1e-13, "page example vs library")
    _close(lse, lse_t, 1e-13, "page example LSE vs library")
    page = _page_order_f32(q[:, 0], k[:, 0], v[:, 0], scale)
    err = np.max(np.abs(o[:, 0] - page))
    assert err <= g["abs_tolerance_f32"], f"page example vs page's f32 order: {err}"


# ------------------------------------ extended oracle: key ranges, offsets, windows
def _ext(lib, q, k, v, scale, causal, **kw):
    return oracle.attn_ref_ext(q, k, v, scale, causal, lib=lib, nthreads=2, **kw)


def _visible(i, S_k, causal, coff, window, kv_begin, kv_end):
    """The keys row i sees, listed one by one (the definition, no ranges)."""
    keys = []
    for j in range(S_k):
        ok = kv_begin <= j < kv_end
        if causal:
            ok = ok and j <= i + coff
        if window > 0:
            ok = ok and j > i + coff - window
        if ok:
            keys.append(j)
    return keys


def pin_ext_bottom_right_library(lib):
    """Offset S_k - S_q (bottom-right alignment): row i is plain attention
    over the key prefix 0 .. i + S_k - S_q, computed by the library routine
    on that prefix."""
    rng = np.random.default_rng(31)
    for S_q, S_k, D in ((5, 9, 4), (7, 7, 3), (3, 12, 8), (16, 40, 16)):
        q = _randn(rng, 1, 2, S_q, D)
        k = _randn(rng, 1, 2, S_k, D)
        v = _randn(rng, 1, 2, S_k, D + 1)
        scale = 0.6
        o, lse = _ext(lib, q, k, v, scale, True, causal_offset=S_k - S_q)
        for i in range(S_q):
            n = i + S_k - S_q + 1
            o_t, lse_t = _library_sdpa(q[:, :, i:i + 1], k[:, :, :n], v[:, :, :n], scale, False)
            _close(o[:, :, i], o_t[:, :, 0], 1e-12, f"bottom-right {S_q}x{S_k} row {i} O")
            _close(lse[:, :, i], lse_t[:, :, 0], 1e-12, f"bottom-right {S_q}x{S_k} row {i} LSE")


def pin_ext_brute_force(lib):
    """40-digit brute force over the explicitly listed visible keys, for key
    ranges, signed offsets and windows; rows without keys: O = 0, LSE = -inf."""
    rng = np.random.default_rng(32)
    for trial in range(60):
        S_q, S_k = int(rng.integers(1, 7)), int(rng.integers(1, 9))
        D_qk, D_v = int(rng.integers(1, 4)), int(rng.integers(1, 3))
        causal = bool(rng.integers(0, 2))
        coff = int(rng.integers(-3, 5))
        window = int(rng.integers(0, 4))
        kv_begin = int(rng.integers(0, S_k + 1))
        kv_end = int(rng.integers(kv_begin, S_k + 1))
        scale = float(rng.uniform(-1.2, 1.2))
        q = _randn(rng, 1, 1, S_q, D_qk, sigma=1.5)
        k = _randn(rng, 1, 1, S_k, D_qk, sigma=1.5)
        v = _randn(rng, 1, 1, S_k, D_v)
        o, lse = _ext(lib, q, k, v, scale, causal, causal_offset=coff, window=window,
                      kv_begin=kv_begin, kv_end=kv_end)
        for i in range(S_q):
            keys = _visible(i, S_k, causal, coff, window, kv_begin, kv_end)
            tag = (f"ext trial {trial} row {i} ({S_q}x{S_k} c{causal} off{coff} w{window} "
                   f"[{kv_begin},{kv_end}))")
            if not keys:
                assert np.all(o[0, 0, i] == 0.0), tag + ": O of an empty row"
                assert lse[0, 0, i] == -np.inf, tag + ": LSE of an empty row"
                continue
            o_mp, lse_mp = _mp_attention_row(q[0, 0, i], k[0, 0][keys], v[0, 0][keys], scale,
                                             len(keys))
            _close(o[0, 0, i], o_mp, 1e-13, tag + " O")
            _close(lse[0, 0, i], lse_mp, 1e-13, tag + " LSE")


def pin_ext_window_of_one(lib):
    """Causal window of one key: row i sees only key i + offset, so O = V
    there and LSE = its scaled score."""
    rng = np.random.default_rng(33)
    S_q, S_k, D = 9, 12, 5
    q = _randn(rng, 1, 1, S_q, D)
    k = _randn(rng, 1, 1, S_k, D)
    v = _randn(rng, 1, 1, S_k, D)
    for coff in (0, 2, -1):
        o, lse = _ext(lib, q, k, v, 0.7, True, causal_offset=coff, window=1)
        for i in range(S_q):
            j = i + coff
            if 0 <= j < S_k:
                _close(o[0, 0, i], v[0, 0, j], 1e-15, f"window 1 off {coff} row {i}")
                _close(lse[0, 0, i], 0.7 * float(q[0, 0, i] @ k[0, 0, j]), 1e-14,
                       f"window 1 off {coff} row {i} LSE")
            else:
                assert lse[0, 0, i] == -np.inf and np.all(o[0, 0, i] == 0.0)


def pin_ext_partition_merge(lib):
    """Split the keys into consecutive chunks: the merge of the chunks'
    (O, LSE) is the result over all keys, for causal (with offsets) and
    non-causal rows, including chunks some rows see nothing of."""
    rng = np.random.default_rng(34)
    for trial in range(20):
        S_q, S_k = int(rng.integers(1, 30)), int(rng.integers(2, 60))
        causal = bool(rng.integers(0, 2))
        coff = int(rng.integers(-4, 8)) if causal else 0
        q = _randn(rng, 1, 2, S_q, 6)
        k = _randn(rng, 1, 2, S_k, 6)
        v = _randn(rng, 1, 2, S_k, 3)
        cuts = sorted(set(int(x) for x in rng.integers(1, S_k, size=int(rng.integers(1, 5)))))
        bounds = [0] + cuts + [S_k]
        parts = [_ext(lib, q, k, v, 0.45, causal, causal_offset=coff, kv_begin=a, kv_end=b)
                 for a, b in zip(bounds, bounds[1:])]
        o_m, lse_m = oracle.merge_ref([p[0] for p in parts], [p[1] for p in parts])
        o_f, lse_f = _ext(lib, q, k, v, 0.45, causal, causal_offset=coff)
        empty = ~np.isfinite(lse_f)
        assert np.array_equal(empty, ~np.isfinite(lse_m)), f"merge trial {trial}: empty rows"
        _close(o_m[~empty], o_f[~empty], 1e-12, f"merge trial {trial} O")
        _close(lse_m[~empty], lse_f[~empty], 1e-12, f"merge trial {trial} LSE")
        assert np.all(o_m[empty] == 0.0)


def pin_gqa_library(lib):
    """Grouped K/V heads against the library routine's own grouped-head mode
    (torch SDPA, enable_gqa): query head h attends with K/V head
    h // (H / H_kv)."""
    rng = np.random.default_rng(51)
    for B, H, H_kv, S, D, causal in ((1, 6, 2, 9, 4, False), (2, 8, 2, 13, 8, True),
                                     (1, 4, 1, 5, 3, False), (1, 6, 3, 11, 5, True)):
        q = _randn(rng, B, H, S, D)
        k = _randn(rng, B, H_kv, S, D)
        v = _randn(rng, B, H_kv, S, D + 2)
        o, lse = _ext(lib, q, k, v, 0.45, causal)
        Q, K, V = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
        o_t = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=causal,
                                                               scale=0.45, enable_gqa=True)
        _close(o, o_t.numpy(), 1e-12, f"gqa H={H} H_kv={H_kv} causal={causal} O")


def pin_gqa_head_map(lib):
    """V constant per K/V head (head j holds j + 1): every output of query
    head h is exactly h // (H / H_kv) + 1, whatever the scores; and a group's
    query heads with equal Q rows produce equal results."""
    rng = np.random.default_rng(52)
    B, H, H_kv, S_q, S_k, D = 2, 12, 4, 7, 10, 5
    g = H // H_kv
    q = _randn(rng, B, H, S_q, D)
    k = _randn(rng, B, H_kv, S_k, D)
    v = np.broadcast_to(np.arange(1, H_kv + 1, dtype=np.float64)[None, :, None, None],
                        (B, H_kv, S_k, 3)).copy()
    o, _ = _ext(lib, q, k, v, 0.7, True, causal_offset=2)
    for h in range(H):
        assert np.all(np.abs(o[:, h] - (h // g + 1)) < 1e-13), f"head map: head {h}"
    v = _randn(rng, B, H_kv, S_k, 3)
    q[:, 1::g] = q[:, 0::g]       # second head of each group repeats the first's Q
    o, lse = _ext(lib, q, k, v, 0.7, False)
    _close(o[:, 1::g], o[:, 0::g], 0.0, "head map: equal heads O")
    _close(lse[:, 1::g], lse[:, 0::g], 0.0, "head map: equal heads LSE")


def _scaled(lib, q, k, v, qs, ks, qb, kb, causal, **kw):
    return oracle.attn_ref_scaled(q, k, v, qs, ks, qb, kb, causal, lib=lib, **kw)


def pin_scaled_constant_scales(lib):
    """Equal scales everywhere: base-2 attention with Q_scale = a and
    K_scale = b is the plain definition with scale a * b * ln 2."""
    rng = np.random.default_rng(61)
    for B, H, S_q, S_k, D, qb, kb, causal in ((1, 2, 9, 13, 4, 3, 5, False),
                                              (2, 1, 17, 11, 8, 4, 2, True),
                                              (1, 1, 1, 1, 3, 1, 1, False)):
        q, k, v = _randn(rng, B, H, S_q, D), _randn(rng, B, H, S_k, D), _randn(rng, B, H, S_k, 5)
        a, b = 0.37, 1.9
        qs = np.full((B, H, -(-S_q // qb)), a)
        ks = np.full((B, H, -(-S_k // kb)), b)
        o, lse = _scaled(lib, q, k, v, qs, ks, qb, kb, causal)
        o_r, lse_r = _ref(lib, q, k, v, a * b * math.log(2.0), causal)
        _close(o, o_r, 1e-12, f"constant scales {S_q}x{S_k} O")
        _close(lse, lse_r, 1e-12, f"constant scales {S_q}x{S_k} LSE")


def pin_scaled_brute_force(lib):
    """40-digit sums of 2^s over every visible key, with per-block scales
    drawn at random (negative and zero query scales, zero key scales)."""
    rng = np.random.default_rng(62)
    mpmath.mp.dps = 40
    for trial in range(40):
        S_q, S_k, D = int(rng.integers(1, 9)), int(rng.integers(1, 11)), int(rng.integers(1, 5))
        qb, kb = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        causal = bool(rng.integers(0, 2))
        q, k, v = _randn(rng, 1, 1, S_q, D), _randn(rng, 1, 1, S_k, D), _randn(rng, 1, 1, S_k, 2)
        qs = rng.normal(size=(1, 1, -(-S_q // qb))) * 2
        ks = np.abs(rng.normal(size=(1, 1, -(-S_k // kb)))) * 2
        if trial % 5 == 0:
            qs[..., 0] = 0.0
            ks[..., -1] = 0.0
        o, lse = _scaled(lib, q, k, v, qs, ks, qb, kb, causal)
        for i in range(S_q):
            n = min(i + 1, S_k) if causal else S_k
            ws = []
            for j in range(n):
                dot = mpmath.fsum(mpmath.mpf(float(q[0, 0, i, d])) * mpmath.mpf(float(k[0, 0, j, d]))
                              for d in range(D))
                sc = mpmath.mpf(float(qs[0, 0, i // qb])) * mpmath.mpf(float(ks[0, 0, j // kb])) * dot
                ws.append(mpmath.power(2, sc))
            tot = mpmath.fsum(ws)
            for e in range(2):
                ref = mpmath.fsum(w * mpmath.mpf(float(v[0, 0, j, e])) for j, w in enumerate(ws)) / tot
                assert abs(float(ref) - o[0, 0, i, e]) <= 1e-12, f"scaled brute force O {trial}"
            assert abs(float(mpmath.log(tot)) - lse[0, 0, i]) <= 1e-12, f"scaled brute force LSE {trial}"


def pin_scaled_zero_key_scales(lib):
    """Every K scale 0: every score is 0, so O is the mean of the visible V
    rows and LSE = ln(number of visible keys)."""
    rng = np.random.default_rng(63)
    S_q, S_k, D = 7, 10, 3
    q, k, v = _randn(rng, 1, 2, S_q, D), _randn(rng, 1, 2, S_k, D), _randn(rng, 1, 2, S_k, 4)
    qs = rng.normal(size=(1, 2, 4))
    ks = np.zeros((1, 2, 4))
    for causal in (False, True):
        o, lse = _scaled(lib, q, k, v, qs, ks, 2, 3, causal)
        for i in range(S_q):
            n = min(i + 1, S_k) if causal else S_k
            _close(o[:, :, i], v[:, :, :n].mean(axis=2), 1e-13, "zero key scales O")
            _close(lse[:, :, i], np.full((1, 2), math.log(n)), 1e-13, "zero key scales LSE")


PINS = [
    pin_library_sdpa,
    pin_highprec_unshifted,
    pin_single_key,
    pin_uniform_weights,
    pin_first_causal_query,
    pin_two_keys,
    pin_far_scores,
    pin_weights_sum_to_one,
    pin_key_permutation,
    pin_score_shift,
    pin_linear_in_v,
    pin_causal_prefix,
    pin_head_dim_padding,
    pin_rows_and_threads,
    pin_page_worked_example,
    pin_ext_bottom_right_library,
    pin_ext_brute_force,
    pin_ext_window_of_one,
    pin_ext_partition_merge,
    pin_gqa_library,
    pin_gqa_head_map,
    pin_scaled_constant_scales,
    pin_scaled_brute_force,
    pin_scaled_zero_key_scales,
]
