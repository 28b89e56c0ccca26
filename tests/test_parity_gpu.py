"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Inputs are seeded and synthetic (tiled_scaled_dot_amd.workloads); the oracle
receives exactly the dtype-rounded values the GPU gets.  Tolerances on the
max absolute error over every active output element:
  O:   1e-4 for f32 inputs, 2e-2 for bf16/f16 inputs (the target's bar);
  LSE: 1e-4 for f32 inputs, 1e-3 for bf16/f16 inputs (our own choice: the
       LSE only sees f32 score/sum rounding, so it is far tighter than O).
Full-size workloads compare a row sample (every 17th row, which visits all
32 row positions of a wave, rows 0, 1, S_q-1, and both sides of every
128-row block boundary); rows are independent, so each sampled row is an
exact check.  The 16-bit workloads of up to 2^31 query-key pairs, and the
long-sequence causal workload with the wide score spread, are also checked
on every row.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_scaled_dot_amd as tsd
from tiled_scaled_dot_amd.workloads import WORKLOADS, make_inputs, random_inputs, sample_rows

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}
TOL_LSE = {"f32": 1e-4, "f16": 1e-3, "bf16": 1e-3}
DEV = "cuda:0"


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(q, k, v, scale, causal, **kw):
    o, lse = tsd.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=causal, **kw)
    torch.cuda.synchronize()
    return o, lse


def run_oracle(q, k, v, scale, causal, rows=None):
    return oracle.attn_ref(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                           scale, causal, rows=rows)


def check(o, lse, o_ref, lse_ref, dtype, what):
    o, lse = np.asarray(o), np.asarray(lse)
    assert np.isfinite(o).all(), f"{what}: non-finite O"
    assert np.isfinite(lse).all(), f"{what}: non-finite LSE"
    err_o = float(np.max(np.abs(o - o_ref)))
    err_l = float(np.max(np.abs(lse - lse_ref)))
    print(f"[parity] {what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= TOL_O[dtype], f"{what}: O error {err_o:.3e} > {TOL_O[dtype]}"
    assert err_l <= TOL_LSE[dtype], f"{what}: LSE error {err_l:.3e} > {TOL_LSE[dtype]}"


# ------------------------------------------------------------ the workloads
SMALL = [n for n, w in WORKLOADS.items() if w.dtype == "f32"]
LARGE = [n for n, w in WORKLOADS.items() if w.dtype != "f32"]


@pytest.mark.parametrize("name", SMALL)
def test_workload_full(name):
    w = WORKLOADS[name]
    print(f"[case] {name}", flush=True)
    q, k, v = make_inputs(w)
    o, lse = run_gpu(q, k, v, w.scale, w.causal)
    o_ref, lse_ref = run_oracle(q, k, v, w.scale, w.causal)
    check(to_np(o), to_np(lse), o_ref, lse_ref, w.dtype, name)


@pytest.mark.parametrize("name", LARGE)
def test_workload_sampled_rows(name):
    w = WORKLOADS[name]
    print(f"[case] {name}", flush=True)
    q, k, v = make_inputs(w)
    o, lse = run_gpu(q, k, v, w.scale, w.causal)
    rows = sample_rows(w.S_q)
    o_s, lse_s = to_np(o[:, :, rows]), to_np(lse[:, :, rows])
    del o, lse
    o_ref, lse_ref = run_oracle(q, k, v, w.scale, w.causal, rows=rows)
    check(o_s, lse_s, o_ref, lse_ref, w.dtype, f"{name} ({len(rows)} rows/slice)")


FULL_16BIT = [n for n in LARGE if WORKLOADS[n].B * WORKLOADS[n].H * WORKLOADS[n].S_q
              * WORKLOADS[n].S_k <= 2 ** 31]


@pytest.mark.parametrize("name", FULL_16BIT)
def test_workload_every_row(name):
    """The 16-bit workloads whose oracle finishes in seconds (up to 2^31
    query-key pairs), every output row checked."""
    w = WORKLOADS[name]
    print(f"[case] {name} (every row)", flush=True)
    q, k, v = make_inputs(w)
    o, lse = run_gpu(q, k, v, w.scale, w.causal)
    o_ref, lse_ref = run_oracle(q, k, v, w.scale, w.causal)
    check(to_np(o), to_np(lse), o_ref, lse_ref, w.dtype, f"{name} (every row)")


def test_long_causal_wide_spread_every_row():
    """bf16 causal, 1 x 32 x 16384 x 128 with Q, K ~ N(0, 3): every one of
    the 524288 output rows against the oracle (about 2.2e12 fp64 FLOP on the
    host, 20-45 s).  Its peaked rows stress the running max hardest."""
    name = "bf16_b1h32_s16384_d128_causal_var3"
    w = WORKLOADS[name]
    print(f"[case] {name} (every row)", flush=True)
    q, k, v = make_inputs(w)
    o, lse = run_gpu(q, k, v, w.scale, w.causal)
    o_np, lse_np = to_np(o), to_np(lse)
    del o, lse
    o_ref, lse_ref = run_oracle(q, k, v, w.scale, w.causal)
    check(o_np, lse_np, o_ref, lse_ref, w.dtype, f"{name} (every row)")


# ------------------------------------------------------------- edge cases
EDGE = [
    # B, H, S_q, S_k, D_qk, D_v, scale
    (1, 1, 1, 1, 1, 1, 0.5),
    (1, 1, 1, 300, 64, 64, 0.125),
    (1, 1, 300, 1, 64, 64, 0.125),
    (2, 3, 129, 65, 64, 64, 0.125),
    (1, 2, 257, 200, 80, 48, 1 / math.sqrt(80)),
    (1, 1, 100, 100, 33, 17, 0.2),
    (1, 1, 70, 50, 1, 1, 1.0),
    (1, 2, 130, 1000, 128, 128, 1 / math.sqrt(128)),
    (1, 2, 1000, 130, 128, 128, 1 / math.sqrt(128)),
    (2, 2, 200, 333, 64, 128, 0.125),
    (2, 2, 200, 333, 128, 64, 1 / math.sqrt(128)),
    (1, 2, 64, 64, 127, 127, 0.09),
    (1, 2, 96, 96, 65, 65, 0.12),
    (1, 2, 96, 96, 96, 96, 0.1),
    (1, 1, 150, 150, 64, 64, -0.3),
    (1, 1, 150, 150, 64, 64, 0.0),
    (1, 1, 150, 150, 32, 32, 0.6),
    (1, 4, 1500, 1500, 64, 64, 0.125),
    (2, 2, 700, 1100, 32, 64, 0.2),
]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", EDGE, ids=[f"{c[0]}x{c[1]}x{c[2]}x{c[3]}_d{c[4]}_{c[5]}_s{c[6]:.3g}"
                                            for c in EDGE])
def test_edge_shapes(case, causal, dtype):
    B, H, S_q, S_k, D_qk, D_v, scale = case
    print(f"[case] {case} causal={causal} {dtype}", flush=True)
    q, k, v = random_inputs((B, H, S_q, D_qk), (B, H, S_k, D_qk), (B, H, S_k, D_v), dtype,
                            seed=1000 + S_q + 7 * S_k + D_qk)
    o, lse = run_gpu(q, k, v, scale, causal)
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal)
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, f"{case} c={causal} {dtype}")


# ------------------------------------ causal key-tile counts, 8-wave shape
@pytest.mark.parametrize("n_tiles", list(range(1, 10)))
def test_causal_tile_counts(n_tiles):
    """Causal bf16 attention at D = 128 over 1-9 key tiles of 64 (ragged by
    13 keys): the causal launches of the 8-wave shape synchronise every
    second tile and split each pair's loads over two tiles, so odd and even
    tile counts, and counts below the ring depth, take different ends of
    the loop."""
    S = 64 * n_tiles - 13
    print(f"[case] causal tiles={n_tiles} S={S}", flush=True)
    q, k, v = random_inputs((1, 2, S + 200, 128), (1, 2, S, 128), (1, 2, S, 128), "bf16",
                            seed=6000 + n_tiles)
    o, lse = run_gpu(q, k, v, 1 / math.sqrt(128), True)
    o_ref, lse_ref = run_oracle(q, k, v, 1 / math.sqrt(128), True)
    check(to_np(o), to_np(lse), o_ref, lse_ref, "bf16", f"causal tiles={n_tiles}")
    # the extended kernel, causal at the bottom right (query i sees keys
    # j <= i + S_k - S_q), S_q = S_k - 40
    qe = q[:, :, : max(S - 40, 1)].contiguous()
    off = S - qe.shape[2]
    o, lse = tsd.attn_fwd_ext(qe.to(DEV), k.to(DEV), v.to(DEV), scale=1 / math.sqrt(128),
                              causal=True, causal_offset=off)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_ref_ext(qe.double().numpy(), k.double().numpy(),
                                         v.double().numpy(), 1 / math.sqrt(128), True,
                                         causal_offset=off)
    check(to_np(o), to_np(lse), o_ref, lse_ref, "bf16", f"ext causal tiles={n_tiles}")


# ------------------------------------------------------ the two f32 kernels
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [
    (2, 16, 2048, 1999, 80, 72),   # 512 blocks of 128 rows: the 128-row kernel
    (2, 16, 1920, 2001, 80, 72),   # 480 such blocks: the key-split kernel
])
def test_f32_kernels_on_large_grids(shape, causal):
    """f32 just above and just below the switch to the key-split kernel (32
    rows per workgroup, the waves splitting the key tiles), a row sample on
    both sides of every block boundary against the oracle."""
    B, H, S_q, S_k, D_qk, D_v = shape
    plan = tsd.attn_fwd_plan(B, H, S_q, S_k, D_qk, D_v, causal, "f32")
    assert plan.key_split == (1 if S_q == 2048 else 4)
    print(f"[case] f32 {shape} causal={causal} block_m={plan.block_m}", flush=True)
    q, k, v = random_inputs((B, H, S_q, D_qk), (B, H, S_k, D_qk), (B, H, S_k, D_v), "f32",
                            seed=5000 + S_q)
    scale = 1 / math.sqrt(D_qk)
    o, lse = run_gpu(q, k, v, scale, causal)
    rows = sample_rows(S_q, block_m=plan.block_m)
    o_s, lse_s = to_np(o[:, :, rows]), to_np(lse[:, :, rows])
    del o, lse
    o_ref, lse_ref = run_oracle(q, k, v, scale, causal, rows=rows)
    check(o_s, lse_s, o_ref, lse_ref, "f32", f"f32 {shape} c={causal} ({len(rows)} rows/slice)")


# ------------------------------------------- masked keys and the running max
def _aligned_inputs(S_q, S_k, D, key_score, dtype, seed):
    """Q rows all equal to u = (1/8, ..., 1/8) and K row j = u * a_j, so that
    with D = 64 and scale 1 the score of every query against key j is a_j;
    V is N(0, 1)."""
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    g = torch.Generator(device="cpu").manual_seed(seed)
    u = torch.full((D,), 1.0 / 8.0)
    a = torch.tensor([key_score(j) for j in range(S_k)], dtype=torch.float64).float()
    q = u.expand(1, 1, S_q, D).clone().to(dt)
    k = (a[:, None] * u[None, :] * (64.0 / D)).reshape(1, 1, S_k, D).to(dt)
    v = torch.randn((1, 1, S_k, D), generator=g).to(dt)
    return q, k, v


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("S_q,S_k", [(700, 700), (700, 650), (130, 1000)])
def test_hidden_keys_never_set_the_max(dtype, S_q, S_k):
    """Causal: scores rise by 2 per key inside every aligned run of 128 keys,
    so for a query at the start of a 64-key tile a later key of that tile
    that leaked into the running max would push its visible exp(s - m)
    below the f32 range (O and LSE would be NaN or far off)."""
    print(f"[case] rising scores causal {S_q}x{S_k} {dtype}", flush=True)
    q, k, v = _aligned_inputs(S_q, S_k, 64, lambda j: 2.0 * (j % 128), dtype, 11)
    o, lse = run_gpu(q, k, v, 1.0, True)
    o_ref, lse_ref = run_oracle(q, k, v, 1.0, True)
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, f"rising causal {S_q}x{S_k} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("S_q,S_k", [(300, 1000), (300, 97), (64, 33)])
def test_keys_past_sk_never_set_the_max(dtype, S_q, S_k):
    """Non-causal, every real score between -206 and -200: the zero-filled
    rows past S_k in the last key tile would score 0 and, if they reached the
    running max, underflow every exp(s - m) to zero."""
    print(f"[case] negative scores {S_q}x{S_k} {dtype}", flush=True)
    q, k, v = _aligned_inputs(S_q, S_k, 64, lambda j: -200.0 - (j % 7), dtype, 12)
    o, lse = run_gpu(q, k, v, 1.0, False)
    o_ref, lse_ref = run_oracle(q, k, v, 1.0, False)
    check(to_np(o), to_np(lse), o_ref, lse_ref, dtype, f"negative {S_q}x{S_k} {dtype}")


# ------------------------------------------------ writes, determinism, streams
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("offset_elems", [0, 1])
def test_no_writes_outside_outputs(dtype, offset_elems):
    """O and LSE sit inside NaN-poisoned buffers with guard bands; an odd
    element offset also disables 16-byte I/O (per-element path)."""
    B, H, S_q, S_k, D_qk, D_v = 2, 3, 200, 150, 80, 72
    q, k, v = random_inputs((B, H, S_q, D_qk), (B, H, S_k, D_qk), (B, H, S_k, D_v), dtype, 77)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    guard = 256 + offset_elems
    n_o, n_l = B * H * S_q * D_v, B * H * S_q
    o_buf = torch.full((n_o + 2 * guard,), float("nan"), dtype=dt, device=DEV)
    l_buf = torch.full((n_l + 2 * 64,), float("nan"), dtype=torch.float32, device=DEV)
    o_view = o_buf[guard:guard + n_o].view(B, H, S_q, D_v)
    l_view = l_buf[64:64 + n_l].view(B, H, S_q)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    if offset_elems:
        # shift the inputs by one element as well
        def shifted(t):
            buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
            view = buf[1:].view(t.shape)
            view.copy_(t)
            return view
        qd, kd, vd = shifted(qd), shifted(kd), shifted(vd)
    tsd.attn_fwd(qd, kd, vd, scale=0.11, causal=True, out=o_view, lse=l_view)
    torch.cuda.synchronize()
    assert torch.isnan(o_buf[:guard]).all() and torch.isnan(o_buf[guard + n_o:]).all()
    assert torch.isnan(l_buf[:64]).all() and torch.isnan(l_buf[64 + n_l:]).all()
    o_ref, lse_ref = run_oracle(q, k, v, 0.11, True)
    check(to_np(o_view), to_np(l_view), o_ref, lse_ref, dtype, f"guard bands {dtype}+{offset_elems}")


def test_bitwise_deterministic():
    w = WORKLOADS["bf16_b4h16_s4096_d128_causal"].with_(B=1, H=8, S_q=1500, S_k=1500)
    q, k, v = (t.to(DEV) for t in make_inputs(w))
    o1, l1 = tsd.attn_fwd(q, k, v, scale=w.scale, causal=True)
    o2, l2 = tsd.attn_fwd(q, k, v, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_non_default_stream():
    w = WORKLOADS["f16_b4h16_q2048_k8192_dqk64_dv128"].with_(B=1, H=8, S_q=700, S_k=900)
    q, k, v = (t.to(DEV) for t in make_inputs(w))
    o1, l1 = tsd.attn_fwd(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o2, l2 = tsd.attn_fwd(q, k, v, scale=w.scale)
    s.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3 = torch.empty_like(o1)
    l3 = torch.empty_like(l1)
    tsd.attn_fwd(q, k, v, scale=w.scale, out=o3, lse=l3, stream=s)
    s.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_lse_optional():
    q, k, v = random_inputs((1, 2, 90, 64), (1, 2, 70, 64), (1, 2, 70, 64), "bf16", 5)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o = torch.empty((1, 2, 90, 64), dtype=torch.bfloat16, device=DEV)
    st = tsd.attn_fwd_raw(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), None,
                          1, 2, 90, 70, 64, 64, 0.125, True, "bf16",
                          torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    o_ref, _ = run_oracle(q, k, v, 0.125, True)
    assert float(np.max(np.abs(to_np(o) - o_ref))) <= TOL_O["bf16"]


# ---------------------------------------------------------- closed forms
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_closed_forms_on_gpu(dtype):
    """Single key -> O = V[0]; Q = 0 -> mean of the visible V rows; the first
    causal query -> V[0]; LSE = ln(number of visible keys) when Q = 0."""
    def same(a, b):
        # 16-bit outputs round the single weight (1 + a few f32 ulp) back to
        # exactly V; f32 outputs keep those last bits.
        if dtype == "f32":
            np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-6)
        else:
            assert np.array_equal(a, b)

    q, k, v = random_inputs((2, 2, 300, 64), (2, 2, 1, 64), (2, 2, 1, 64), dtype, 3)
    o, lse = run_gpu(q, k, v, 0.2, False)
    same(to_np(o), np.broadcast_to(to_np(v), o.shape))
    q, k, v = random_inputs((1, 2, 200, 64), (1, 2, 150, 64), (1, 2, 150, 64), dtype, 4)
    o, lse = run_gpu(torch.zeros_like(q), k, v, 0.2, True)
    vv = v.double().numpy()
    counts = np.minimum(np.arange(200) + 1, 150)
    means = np.cumsum(vv, axis=2)[:, :, counts - 1] / counts[None, None, :, None]
    check(to_np(o), to_np(lse), means, np.broadcast_to(np.log(counts), (1, 2, 200)), dtype,
          f"Q=0 causal prefix mean {dtype}")
    o, _ = run_gpu(q, k, v, 0.2, True)
    same(to_np(o[:, :, 0]), to_np(v[:, :, 0]))


def test_page_worked_example_on_gpu():
    from oracle_pins import load_page_example
    g, q, k, v = load_page_example()
    tq, tk, tv = (torch.from_numpy(x).float() for x in (q, k, v))
    scale = 1.0 / math.sqrt(g["qk"])
    o, lse = run_gpu(tq, tk, tv, scale, False)
    o_ref, lse_ref = run_oracle(tq, tk, tv, scale, False)
    check(to_np(o), to_np(lse), o_ref, lse_ref, "f32", "page worked example")
    assert float(np.max(np.abs(to_np(o) - o_ref))) <= g["abs_tolerance_f32"]
