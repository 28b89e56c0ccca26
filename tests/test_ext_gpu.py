"""GPU parity of the extended entry points against the fp64 oracle.

attn_fwd_ext (causal offset, sliding window, key range), attn_fwd_partial
(one result per key chunk), attn_merge (the continuation pass) and
attn_fwd_splitkv (partial + merge), all through the C ABI, compared with
oracle.attn_ref_ext / oracle.merge_ref on the same seeded inputs.

Tolerances are those of the plain path (O: 2e-2 for 16-bit inputs, 1e-4
for f32; LSE: 1e-3 / 1e-4).  A row that sees no key must come back exactly
as O = 0 and LSE = -inf.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_scaled_dot_amd as tsd
from tiled_scaled_dot_amd.workloads import random_inputs, sample_rows

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}
TOL_LSE = {"f32": 1e-4, "f16": 1e-3, "bf16": 1e-3}
DEV = "cuda:0"


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(o, lse, o_ref, lse_ref, dtype, what, tol_o=None, tol_l=None):
    """Max-abs comparison; rows whose reference LSE is -inf must be exactly
    O = 0, LSE = -inf on the GPU too."""
    o, lse = np.asarray(o), np.asarray(lse)
    tol_o = TOL_O[dtype] if tol_o is None else tol_o
    tol_l = TOL_LSE[dtype] if tol_l is None else tol_l
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty rows differ"
    assert np.all(o[empty] == 0.0), f"{what}: empty row with nonzero O"
    live = ~empty
    assert np.isfinite(o[live]).all() and np.isfinite(lse[live]).all(), f"{what}: non-finite"
    err_o = float(np.max(np.abs(o[live] - o_ref[live]))) if live.any() else 0.0
    err_l = float(np.max(np.abs(lse[live] - lse_ref[live]))) if live.any() else 0.0
    print(f"[parity] {what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} "
          f"empty rows={int(empty.sum())}", flush=True)
    assert err_o <= tol_o, f"{what}: O error {err_o:.3e} > {tol_o}"
    assert err_l <= tol_l, f"{what}: LSE error {err_l:.3e} > {tol_l}"


def ref_ext(q, k, v, scale, causal, coff=0, window=0, kv_begin=0, kv_end=None, rows=None):
    return oracle.attn_ref_ext(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                               scale, causal, causal_offset=coff, window=window,
                               kv_begin=kv_begin, kv_end=kv_end, rows=rows)


def gpu(*ts):
    return [t.to(DEV) for t in ts]


# ------------------------------------------------------------ attn_fwd_ext
MASKS = [
    # B, H, S_q, S_k, D_qk, D_v, causal, causal_offset, window, kv_begin, kv_end
    (1, 2, 300, 1000, 128, 128, True, 700, 0, 0, None),      # bottom-right diagonal
    (1, 2, 300, 1000, 64, 64, True, 700, 0, 0, None),
    (1, 2, 700, 700, 128, 128, True, -150, 0, 0, None),      # rows 0..149 see nothing
    (1, 2, 700, 700, 64, 64, True, -150, 0, 0, None),
    (1, 2, 1100, 1100, 128, 128, True, 0, 200, 0, None),     # sliding window
    (1, 2, 1100, 1100, 64, 64, True, 0, 200, 0, None),
    (1, 2, 1100, 1100, 128, 128, True, 0, 1, 0, None),       # window of one key
    (1, 2, 600, 900, 128, 128, False, 0, 300, 0, None),      # window, no upper bound
    (2, 2, 500, 1500, 64, 128, True, 1000, 333, 0, None),    # offset + window, D_qk != D_v
    (1, 2, 800, 1000, 128, 64, False, 0, 0, 130, 900),       # key range
    (1, 2, 800, 1000, 128, 128, True, 0, 0, 130, 900),
    (1, 2, 800, 1000, 128, 128, True, 100, 77, 130, 900),    # all of them
    (1, 1, 200, 300, 64, 64, False, 0, 0, 64, 64),           # empty key range
    (1, 3, 129, 65, 64, 64, True, 0, 5, 0, None),            # ragged and tiny
    (2, 8, 256, 4096, 128, 128, True, 3840, 1024, 0, None),  # 16 slices (XCD order)
    (1, 2, 1000, 777, 80, 80, True, -300, 250, 0, None),     # head-dim tail, ragged S_k
]


def mask_id(c):
    B, H, S_q, S_k, dq, dv, causal, coff, win, kb, ke = c
    return f"{B}x{H}x{S_q}x{S_k}_d{dq}-{dv}_c{int(causal)}_off{coff}_w{win}_kv{kb}-{ke}"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", MASKS, ids=[mask_id(c) for c in MASKS])
def test_ext_masks(case, dtype):
    B, H, S_q, S_k, D_qk, D_v, causal, coff, window, kb, ke = case
    print(f"[case] ext {mask_id(case)} {dtype}", flush=True)
    scale = 1 / math.sqrt(D_qk)
    q, k, v = random_inputs((B, H, S_q, D_qk), (B, H, S_k, D_qk), (B, H, S_k, D_v), dtype,
                            seed=2000 + S_q + 3 * S_k + coff + window)
    o, lse = tsd.attn_fwd_ext(*gpu(q, k, v), scale=scale, causal=causal, causal_offset=coff,
                              window=window, kv_begin=kb, kv_end=ke)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_ext(q, k, v, scale, causal, coff, window, kb, ke)
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, f"ext {mask_id(case)} {dtype}")


# Slices of at most 32 query rows (decoding): one wave holds every row and
# the others only stream tiles.  The cases put the visible keys in one half
# of a 64-key tile (S_k or the window under 32, a key range inside one
# half), make some rows see nothing, and cover the head widths of both
# launch shapes.
DECODE = [
    # B, H, S_q, S_k, D_qk, D_v, causal, causal_offset, window, kv_begin, kv_end
    (2, 4, 1, 1, 128, 128, True, 0, 0, 0, None),             # one key: the second half is empty
    (2, 4, 1, 31, 128, 128, True, 30, 0, 0, None),           # keys in the first half only
    (1, 4, 1, 33, 64, 64, True, 32, 0, 0, None),             # one key in the second half
    (1, 4, 1, 4097, 128, 128, True, 4096, 0, 0, None),
    (2, 3, 7, 1000, 128, 128, True, 993, 0, 0, None),
    (1, 2, 32, 2000, 64, 64, True, 1968, 0, 0, None),        # 32 rows: the largest such slice
    (1, 2, 31, 777, 80, 80, True, 746, 0, 0, None),          # head-width tail
    (1, 2, 16, 900, 64, 128, True, 884, 0, 0, None),         # D_qk != D_v
    (1, 2, 16, 900, 128, 64, False, 0, 0, 0, None),
    (1, 2, 20, 1000, 128, 128, True, -10, 0, 0, None),       # rows 0..9 see nothing
    (1, 2, 5, 3000, 128, 128, True, 2995, 20, 0, None),      # window inside one half
    (1, 2, 5, 3000, 128, 128, True, 2995, 40, 0, None),      # window across both halves
    (1, 2, 5, 3000, 64, 64, True, 2995, 1000, 0, None),
    (1, 2, 8, 2000, 128, 128, False, 0, 0, 96, 120),          # key range in the second half
    (1, 2, 8, 2000, 128, 128, False, 0, 0, 64, 90),           # ... in the first half
    (1, 2, 8, 2000, 128, 128, True, 1500, 100, 130, 1900),
    (1, 1, 4, 300, 64, 64, False, 0, 0, 64, 64),              # empty key range
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", DECODE, ids=[mask_id(c) for c in DECODE])
def test_ext_decode_rows(case, dtype):
    B, H, S_q, S_k, D_qk, D_v, causal, coff, window, kb, ke = case
    print(f"[case] ext decode {mask_id(case)} {dtype}", flush=True)
    scale = 1 / math.sqrt(D_qk)
    q, k, v = random_inputs((B, H, S_q, D_qk), (B, H, S_k, D_qk), (B, H, S_k, D_v), dtype,
                            seed=2500 + S_q + 3 * S_k + coff + window)
    o, lse = tsd.attn_fwd_ext(*gpu(q, k, v), scale=scale, causal=causal, causal_offset=coff,
                              window=window, kv_begin=kb, kv_end=ke)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_ext(q, k, v, scale, causal, coff, window, kb, ke)
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, f"ext decode {mask_id(case)} {dtype}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 4, 1000, 777, 128, 128), (1, 2, 513, 1029, 64, 64),
                                   (2, 8, 384, 640, 64, 128), (1, 1, 1, 200, 128, 64)])
def test_ext_default_mask_is_attn_fwd(shape, causal):
    """With the default mask the extended kernel takes the same decisions in
    the same order as the plain one: the results are bit-identical."""
    B, H, S_q, S_k, D_qk, D_v = shape
    print(f"[case] ext==fwd {shape} causal={causal}", flush=True)
    q, k, v = gpu(*random_inputs((B, H, S_q, D_qk), (B, H, S_k, D_qk), (B, H, S_k, D_v),
                                 "bf16", seed=77 + S_q))
    o1, l1 = tsd.attn_fwd(q, k, v, causal=causal)
    o2, l2 = tsd.attn_fwd_ext(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_ext_window_of_one_returns_v():
    """Window 1 with the causal diagonal: row i sees only key i, so O = V[i]
    (to the output rounding) and LSE = scale * q_i . k_i."""
    q, k, v = random_inputs((1, 2, 300, 64), (1, 2, 300, 64), (1, 2, 300, 64), "bf16", seed=5)
    o, lse = tsd.attn_fwd_ext(*gpu(q, k, v), scale=0.125, causal=True, window=1)
    torch.cuda.synchronize()
    assert torch.equal(o.cpu(), v)
    s = 0.125 * (q.double() * k.double()).sum(-1)
    assert float((lse.cpu().double() - s).abs().max()) <= 1e-3


# --------------------------------------------------------- attn_fwd_partial
PARTIALS = [
    # B, H, S_q, S_k, D, causal, coff, window, kv_begin, kv_end, n_splits, split_len
    (1, 2, 300, 2000, 128, False, 0, 0, 0, None, 4, 512),
    (1, 2, 300, 2000, 128, True, 1700, 0, 0, None, 5, 448),
    (1, 2, 300, 2000, 64, True, 1700, 600, 0, None, 8, 256),   # chunks empty for all rows
    (1, 2, 300, 2000, 128, False, 0, 0, 100, 1900, 3, 700),    # chunks not on tile bounds
    (1, 1, 100, 500, 64, False, 0, 0, 0, None, 6, 128),        # chunks past the range
    (2, 4, 1, 5000, 128, True, 4999, 0, 0, None, 7, 768),     # one row per slice
    (1, 2, 24, 3000, 64, True, 2976, 500, 0, None, 4, 832),   # 24 rows, window
    (2, 8, 256, 3000, 128, True, 2744, 0, 0, None, 3, 1024),   # 16 slices
]


@pytest.mark.parametrize("case", PARTIALS, ids=[f"p{i}" for i in range(len(PARTIALS))])
def test_partial_chunks(case):
    B, H, S_q, S_k, D, causal, coff, window, kb, ke, n, ln = case
    print(f"[case] partial {case}", flush=True)
    ke_ = S_k if ke is None else ke
    scale = 1 / math.sqrt(D)
    q, k, v = random_inputs((B, H, S_q, D), (B, H, S_k, D), (B, H, S_k, D), "bf16",
                            seed=3000 + S_k + n)
    op, lp = tsd.attn_fwd_partial(*gpu(q, k, v), n, ln, scale=scale, causal=causal,
                                  causal_offset=coff, window=window, kv_begin=kb, kv_end=ke)
    torch.cuda.synchronize()
    op, lp = to_np(op), to_np(lp)
    for s in range(n):
        lo = min(kb + s * ln, ke_)
        hi = min(ke_, kb + (s + 1) * ln)
        o_ref, lse_ref = ref_ext(q, k, v, scale, causal, coff, window, lo, max(lo, hi))
        # f32 partial output: only the 16-bit P rounding, tolerance of 16-bit inputs
        check(op[s], lp[s], o_ref, lse_ref, "bf16", f"partial {case} chunk {s}")
    # the merge of the chunks is the whole range
    o_ref, lse_ref = ref_ext(q, k, v, scale, causal, coff, window, kb, ke)
    o_m, l_m = oracle.merge_ref(op, lp)
    check(o_m, l_m, o_ref, lse_ref, "bf16", f"partial {case} merged on the host")


# --------------------------------------------------------------- attn_merge
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n,D_v", [(1, 128), (3, 128), (17, 64), (4, 37), (2, 5)])
def test_merge(n, D_v, dtype):
    print(f"[case] merge n={n} D_v={D_v} {dtype}", flush=True)
    B, H, S_q = 2, 3, 77
    g = torch.Generator().manual_seed(40 + n * 7 + D_v)
    o_parts = torch.randn((n, B, H, S_q, D_v), generator=g)
    lse_parts = torch.randn((n, B, H, S_q), generator=g) * 4.0
    # some chunks see nothing (-inf), and rows 0 and 5 of every slice none at all
    drop = torch.rand((n, B, H, S_q), generator=g) < 0.3
    lse_parts[drop] = -math.inf
    o_parts[drop] = 0.0
    lse_parts[:, :, :, 0] = -math.inf
    lse_parts[:, :, :, 5] = -math.inf
    o_parts[:, :, :, 0] = 0.0
    o_parts[:, :, :, 5] = 0.0
    out_dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    o, lse = tsd.attn_merge(o_parts.to(DEV), lse_parts.to(DEV), dtype=out_dt)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.merge_ref(o_parts.double().numpy(), lse_parts.double().numpy())
    # the 16-bit output rounds O (|O| < ~4): bf16 half-ulp <= 2^-7 * 4
    tol_o = {"f32": 1e-5, "bf16": 2e-2, "f16": 4e-3}[dtype]
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, f"merge n={n} D_v={D_v} {dtype}",
          tol_o=tol_o, tol_l=1e-5)


# --------------------------------------------------------- attn_fwd_splitkv
SPLITS = [
    # B, H, S_q, S_k, D_qk, D_v, causal, coff, window, n_splits
    (1, 4, 256, 8192, 128, 128, False, 0, 0, 0),
    (1, 4, 256, 8192, 128, 128, True, 7936, 0, 0),
    (2, 2, 100, 5000, 64, 64, False, 0, 0, 7),
    (1, 2, 64, 3000, 128, 128, True, 2936, 1000, 5),
    (1, 8, 1, 20000, 128, 128, True, 19999, 0, 0),      # one query row: decoding
    (1, 2, 2048, 2048, 128, 128, True, 0, 0, 0),        # the plan keeps one chunk
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", SPLITS, ids=[f"s{i}" for i in range(len(SPLITS))])
def test_splitkv(case, dtype):
    B, H, S_q, S_k, D_qk, D_v, causal, coff, window, n = case
    print(f"[case] splitkv {case} {dtype}", flush=True)
    scale = 1 / math.sqrt(D_qk)
    q, k, v = random_inputs((B, H, S_q, D_qk), (B, H, S_k, D_qk), (B, H, S_k, D_v), dtype,
                            seed=4000 + S_k + S_q)
    plan = tsd.attn_splitkv_plan(B, H, S_q, S_k, D_qk, D_v, causal, dtype,
                                 tsd.make_mask(S_k, coff, window), n)
    print(f"[plan] chunks={plan[0]} keys/chunk={plan[1]} workspace={plan[2]}", flush=True)
    o, lse = tsd.attn_fwd_splitkv(*gpu(q, k, v), scale=scale, causal=causal,
                                  causal_offset=coff, window=window, n_splits=n)
    torch.cuda.synchronize()
    rows = sample_rows(S_q) if S_q > 512 else None
    o_ref, lse_ref = ref_ext(q, k, v, scale, causal, coff, window, rows=rows)
    if rows is not None:
        o, lse = o[:, :, rows], lse[:, :, rows]
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, f"splitkv {case} {dtype}")


def test_splitkv_reuses_workspace():
    """Two calls of different sizes on one workspace: the second result
    carries nothing over from the first."""
    q, k, v = random_inputs((1, 4, 128, 128), (1, 4, 6000, 128), (1, 4, 6000, 128), "bf16",
                            seed=9)
    n, _, ws = tsd.attn_splitkv_plan(1, 4, 128, 6000, 128, 128, False, "bf16", None, 8)
    work = torch.empty(ws, dtype=torch.uint8, device=DEV)
    qg, kg, vg = gpu(q, k, v)
    tsd.attn_fwd_splitkv(qg, kg, vg, n_splits=8, workspace=work)
    o2, l2 = tsd.attn_fwd_splitkv(qg[:, :2, :50].contiguous(), kg[:, :2, :3000].contiguous(),
                                  vg[:, :2, :3000].contiguous(), n_splits=4, workspace=work)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_ext(q[:, :2, :50], k[:, :2, :3000], v[:, :2, :3000],
                             1 / math.sqrt(128), False)
    check(to_np(o2), to_np(l2), o_ref, lse_ref, "bf16", "splitkv reuse")


# ------------------------------------------------------- grouped K/V heads
GQA = [
    # B, H, H_kv, S_q, S_k, D, causal, causal_offset, window
    (1, 8, 2, 300, 700, 128, True, 400, 0),      # a workgroup's rows span two heads
    (2, 6, 3, 129, 257, 64, False, 0, 0),
    (1, 8, 1, 1, 3000, 128, True, 2999, 0),      # one K/V head, one query: decoding
    (2, 32, 8, 1, 4096, 128, True, 4095, 0),
    (1, 4, 2, 200, 600, 64, True, 400, 150),     # window
    (1, 4, 4, 300, 300, 128, True, 0, 0),        # H_kv = H
    (1, 16, 2, 40, 900, 128, True, 860, 64),     # 8 heads of 40 rows per slice
    (1, 8, 2, 8, 1000, 64, True, 992, 0),        # 4 heads of 8 rows: 32 rows per slice
    (1, 12, 4, 10, 700, 128, True, 690, 0),      # 3 heads of 10 rows per slice
]


def gqa_id(c):
    return "gqa_{}x{}kv{}_{}x{}_d{}_c{}_off{}_w{}".format(*(int(x) for x in c))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", GQA, ids=[gqa_id(c) for c in GQA])
def test_gqa_ext(case, dtype):
    B, H, H_kv, S_q, S_k, D, causal, coff, window = case
    print(f"[case] {gqa_id(case)} {dtype}", flush=True)
    scale = 1 / math.sqrt(D)
    q, k, v = random_inputs((B, H, S_q, D), (B, H_kv, S_k, D), (B, H_kv, S_k, D), dtype,
                            seed=5000 + H * 7 + H_kv + S_q)
    o, lse = tsd.attn_fwd_ext(*gpu(q, k, v), scale=scale, causal=causal, causal_offset=coff,
                              window=window)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_ext(q, k, v, scale, causal, coff, window)
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, f"{gqa_id(case)} {dtype}")


@pytest.mark.parametrize("case", [(4, 32, 8, 1, 16384, 128, True, 16383, 0, 0),
                                  (1, 8, 2, 64, 5000, 128, True, 4936, 0, 5),
                                  (2, 4, 1, 3, 3000, 64, False, 0, 0, 3)],
                         ids=["decode_auto", "chunk_n5", "mqa_n3"])
def test_gqa_splitkv(case):
    B, H, H_kv, S_q, S_k, D, causal, coff, window, n = case
    print(f"[case] gqa splitkv {case}", flush=True)
    scale = 1 / math.sqrt(D)
    q, k, v = random_inputs((B, H, S_q, D), (B, H_kv, S_k, D), (B, H_kv, S_k, D), "bf16",
                            seed=6000 + S_k)
    plan = tsd.attn_splitkv_plan(B, H, S_q, S_k, D, D, causal, "bf16",
                                 tsd.make_mask(S_k, coff, window), n, H_kv=H_kv)
    print(f"[plan] chunks={plan[0]} keys/chunk={plan[1]} workspace={plan[2]}", flush=True)
    o, lse = tsd.attn_fwd_splitkv(*gpu(q, k, v), scale=scale, causal=causal,
                                  causal_offset=coff, window=window, n_splits=n)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_ext(q, k, v, scale, causal, coff, window)
    check(to_np(o), to_np(lse), o_ref, lse_ref, "bf16", f"gqa splitkv {case}")


def test_gqa_partial():
    B, H, H_kv, S_q, S_k, D, n, ln = 1, 6, 2, 50, 1000, 64, 4, 256
    q, k, v = random_inputs((B, H, S_q, D), (B, H_kv, S_k, D), (B, H_kv, S_k, D), "bf16",
                            seed=61)
    op, lp = tsd.attn_fwd_partial(*gpu(q, k, v), n, ln, scale=0.125, causal=True,
                                  causal_offset=S_k - S_q)
    torch.cuda.synchronize()
    op, lp = to_np(op), to_np(lp)
    for s in range(n):
        o_ref, lse_ref = ref_ext(q, k, v, 0.125, True, S_k - S_q, 0, s * ln,
                                 min(S_k, (s + 1) * ln))
        check(op[s], lp[s], o_ref, lse_ref, "bf16", f"gqa partial chunk {s}")


@pytest.mark.parametrize("window", [1, 200, 1000])
def test_window_and_complement_partition_causal(window):
    """The sliding window (the `window` keys ending at the diagonal) and its
    complement (the causal mask moved back by `window`) split every causal
    row's keys in two: merging the two results gives plain causal attention,
    and each part matches the oracle on its own."""
    B, H, S, D = 1, 2, 1500, 128
    q, k, v = random_inputs((B, H, S, D), (B, H, S, D), (B, H, S, D), "bf16", seed=71 + window)
    qg, kg, vg = gpu(q, k, v)
    ow, lw = tsd.attn_fwd_ext(qg, kg, vg, scale=0.09, causal=True, window=window)
    oc, lc = tsd.attn_fwd_ext(qg, kg, vg, scale=0.09, causal=True, causal_offset=-window)
    o_all, l_all = tsd.attn_fwd(qg, kg, vg, scale=0.09, causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = ref_ext(q, k, v, 0.09, True, 0, window)
    check(to_np(ow), to_np(lw), o_ref, l_ref, "bf16", f"window {window}")
    o_ref, l_ref = ref_ext(q, k, v, 0.09, True, -window)
    check(to_np(oc), to_np(lc), o_ref, l_ref, "bf16", f"complement of window {window}")
    # the merge of the two parts on the GPU is the plain causal result
    parts_o = torch.stack([ow.float(), oc.float()])
    parts_l = torch.stack([lw, lc])
    om, lm = tsd.attn_merge(parts_o.contiguous(), parts_l.contiguous(), dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, l_ref = ref_ext(q, k, v, 0.09, True)
    check(to_np(om), to_np(lm), o_ref, l_ref, "bf16", f"window {window} + complement merged")
    check(to_np(o_all), to_np(l_all), o_ref, l_ref, "bf16", "plain causal")


# Keys that no query row of the call sees may hold any bits: they are never
# read into a result.  The cases fill them with NaN (K) and NaN or infinity
# (V): an unwritten cache tail after kv_end, a prefix before kv_begin, the
# keys after the last row's diagonal and before the first row's window.
UNSEEN = [
    # B, H, H_kv, S_q, S_k, D, causal, causal_offset, window, kv_begin, kv_end, entry
    (2, 8, 2, 1, 5000, 128, True, 3000, 0, 0, 3001, "ext"),         # decoding, cache tail
    (2, 8, 2, 1, 5000, 128, True, 3000, 0, 0, 3001, "splitkv"),
    (2, 8, 2, 1, 5000, 128, True, 3000, 0, 0, 3001, "noalloc"),
    (1, 4, 4, 40, 2100, 64, False, 0, 0, 100, 2000, "ext"),         # prefix and tail
    (1, 4, 4, 40, 2100, 64, False, 0, 0, 100, 2000, "splitkv"),
    (1, 2, 2, 300, 1000, 128, True, 500, 200, 0, None, "ext"),      # diagonal and window
    (1, 6, 3, 7, 777, 128, True, 700, 0, 37, 701, "splitkv"),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", UNSEEN, ids=[f"u{i}" for i in range(len(UNSEEN))])
def test_unseen_keys_never_reach_results(case, dtype):
    B, H, H_kv, S_q, S_k, D, causal, coff, window, kb, ke, entry = case
    print(f"[case] unseen keys {case} {dtype}", flush=True)
    q, k, v = random_inputs((B, H, S_q, D), (B, H_kv, S_k, D), (B, H_kv, S_k, D), dtype,
                            seed=7000 + S_k + S_q)
    ke_ = S_k if ke is None else ke
    # keys no row sees: outside [kb, ke), after the last row's diagonal,
    # before the first row's window
    seen_lo = max(kb, coff - window + 1) if window > 0 else kb
    seen_hi = min(ke_, S_q - 1 + coff + 1) if causal else ke_
    unseen = torch.ones(S_k, dtype=torch.bool)
    unseen[seen_lo:seen_hi] = False
    assert unseen.any()
    k[:, :, unseen] = float("nan")
    v[:, :, unseen] = float("nan")
    v[:, :, unseen.nonzero()[::2, 0]] = float("inf")
    scale = 1 / math.sqrt(D)
    kw = dict(scale=scale, causal=causal, causal_offset=coff, window=window, kv_begin=kb,
              kv_end=ke)
    qg, kg, vg = gpu(q, k, v)
    if entry == "ext":
        o, lse = tsd.attn_fwd_ext(qg, kg, vg, **kw)
    elif entry == "splitkv":
        o, lse = tsd.attn_fwd_splitkv(qg, kg, vg, n_splits=3, **kw)
    else:
        o, lse = tsd.attn_fwd_splitkv_noalloc(qg, kg, vg, **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_ext(q, k, v, scale, causal, coff, window, kb, ke)
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, f"unseen keys {case} {dtype}")
