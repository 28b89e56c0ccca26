"""GPU parity of attn_fwd_scaled (base-2 attention with per-block Q/K
scales; fp8 or 16-bit Q and K) against oracle.attn_ref_scaled.

The oracle receives exactly the stored values: fp8 Q/K decoded to float64
(every e4m3 value is exact in float64) and the float32 block scales.
Tolerances as for the plain path with 16-bit inputs: O <= 2e-2, LSE <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_scaled_dot_amd as tsd
from tiled_scaled_dot_amd.workloads import sample_rows, scaled_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL_O, TOL_LSE = 2e-2, 1e-3


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run(q, k, v, qs, ks, qb, kb, causal):
    o, lse = tsd.attn_fwd_scaled(q.to(DEV), k.to(DEV), v.to(DEV), qs.to(DEV), ks.to(DEV), qb,
                                 kb, causal)
    torch.cuda.synchronize()
    return o, lse


def ref(q, k, v, qs, ks, qb, kb, causal, rows=None):
    return oracle.attn_ref_scaled(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                  qs.double().numpy(), ks.double().numpy(), qb, kb, causal,
                                  rows=rows)


def check(o, lse, o_ref, lse_ref, what):
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{what}: non-finite"
    err_o = float(np.max(np.abs(o - o_ref)))
    err_l = float(np.max(np.abs(lse - lse_ref)))
    print(f"[parity] {what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= TOL_O, f"{what}: O error {err_o:.3e}"
    assert err_l <= TOL_LSE, f"{what}: LSE error {err_l:.3e}"


CASES = [
    # B, H, S_q, S_k, D_qk, D_v, q_block, k_block
    (1, 2, 300, 700, 128, 128, 128, 64),
    (2, 2, 257, 513, 64, 64, 64, 128),
    (1, 3, 129, 65, 80, 64, 128, 64),       # head-dim tail, ragged S_k inside one key block
    (1, 2, 1000, 1000, 128, 128, 32, 192),  # query blocks finer than a workgroup
    (1, 1, 1, 64, 128, 128, 1, 64),
    (2, 8, 256, 1024, 128, 128, 256, 256),  # 16 slices (XCD order)
]


def case_id(c):
    return "{}x{}x{}x{}_d{}-{}_qb{}_kb{}".format(*c)


@pytest.mark.parametrize("qk", ["fp8_e4m3", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", CASES, ids=[case_id(c) for c in CASES])
def test_scaled_parity(case, causal, qk):
    B, H, S_q, S_k, D_qk, D_v, qb, kb = case
    vdt = "f16" if qk == "f16" else "bf16"
    print(f"[case] scaled {case_id(case)} causal={causal} qk={qk}", flush=True)
    q, k, v, qs, ks = scaled_inputs(B, H, S_q, S_k, D_qk, D_v, qb, kb, qk, vdt,
                                    seed=7000 + S_q + S_k + D_qk, scale_jitter=True)
    o, lse = run(q, k, v, qs, ks, qb, kb, causal)
    o_ref, lse_ref = ref(q, k, v, qs, ks, qb, kb, causal)
    check(to_np(o), to_np(lse), o_ref, lse_ref, f"{case_id(case)} c={causal} {qk}")


@pytest.mark.parametrize("qk", ["fp8_e4m3", "bf16"])
def test_scaled_special_blocks(qk):
    """A zero and a negative query-block scale, a zero key-block scale."""
    B, H, S_q, S_k, D, qb, kb = 1, 2, 400, 600, 128, 100, 128
    q, k, v, qs, ks = scaled_inputs(B, H, S_q, S_k, D, D, qb, kb, qk, "bf16", seed=77)
    qs[:, :, 1] = 0.0
    qs[:, :, 2] *= -1.0
    ks[:, :, 2] = 0.0
    for causal in (False, True):
        o, lse = run(q, k, v, qs, ks, qb, kb, causal)
        o_ref, lse_ref = ref(q, k, v, qs, ks, qb, kb, causal)
        check(to_np(o), to_np(lse), o_ref, lse_ref, f"special blocks {qk} c={causal}")


NEG_CASES = [
    # B, H, S_q, S_k, D_qk, D_v, q_block, k_block
    (1, 2, 400, 700, 128, 128, 100, 64),
    (2, 2, 257, 513, 64, 64, 64, 128),
    (1, 3, 300, 1000, 128, 128, 128, 192),
]


@pytest.mark.parametrize("qk", ["fp8_e4m3", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pattern", ["all_negative", "mixed", "alternating_zero"])
@pytest.mark.parametrize("case", NEG_CASES, ids=[case_id(c) for c in NEG_CASES])
def test_scaled_negative_key_scales(case, pattern, causal, qk):
    """Key-block scales of either sign (the per-key scale of the definition
    has no sign premise): all negative, a seeded random mix of signs (with
    negative query scales too), and signs alternating with zero scales, so
    that consecutive key tiles switch sign."""
    B, H, S_q, S_k, D_qk, D_v, qb, kb = case
    vdt = "f16" if qk == "f16" else "bf16"
    print(f"[case] negative key scales {case_id(case)} {pattern} causal={causal} qk={qk}",
          flush=True)
    q, k, v, qs, ks = scaled_inputs(B, H, S_q, S_k, D_qk, D_v, qb, kb, qk, vdt,
                                    seed=7500 + S_q + S_k, scale_jitter=True)
    g = torch.Generator(device="cpu").manual_seed(7600 + S_k)
    if pattern == "all_negative":
        ks = -ks
    elif pattern == "mixed":
        ks = ks * torch.where(torch.rand(ks.shape, generator=g) < 0.5, -1.0, 1.0)
        qs = qs * torch.where(torch.rand(qs.shape, generator=g) < 0.3, -1.0, 1.0)
    else:
        sign = torch.tensor([1.0, -1.0, 0.0, -1.0]).repeat(ks.shape[-1] // 4 + 1)
        ks = ks * sign[: ks.shape[-1]]
    ks, qs = ks.contiguous(), qs.contiguous()
    o, lse = run(q, k, v, qs, ks, qb, kb, causal)
    o_ref, lse_ref = ref(q, k, v, qs, ks, qb, kb, causal)
    check(to_np(o), to_np(lse), o_ref, lse_ref,
          f"negative key scales {case_id(case)} {pattern} c={causal} {qk}")


def test_scaled_negated_key_scales_mirror_the_scores():
    """K_scale -> -K_scale gives the attention of -K with the original
    scales: the same scores with their sign flipped, computed two ways."""
    B, H, S, D, qb, kb = 1, 2, 500, 128, 128, 64
    q, k, v, qs, ks = scaled_inputs(B, H, S, S, D, D, qb, kb, "bf16", "bf16", seed=81,
                                    scale_jitter=True)
    for causal in (False, True):
        o1, l1 = run(q, k, v, qs, -ks, qb, kb, causal)
        o2, l2 = run(q, -k, v, qs, ks, qb, kb, causal)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"causal={causal}"


def test_scaled_matches_plain_attention():
    """16-bit Q/K with Q_scale = scale * log2(e) and K_scale = 1 is the plain
    attention of attn_fwd (the same kernel decisions, base 2 either way): the
    two agree to the 16-bit output rounding."""
    B, H, S, D = 1, 2, 700, 128
    q, k, v, qs, ks = scaled_inputs(B, H, S, S, D, D, 64, 64, "bf16", "bf16", seed=78)
    for causal in (False, True):
        o1, l1 = run(q, k, v, qs, ks, 64, 64, causal)
        o2, l2 = tsd.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=1 / math.sqrt(D),
                              causal=causal)
        torch.cuda.synchronize()
        assert float((o1.float() - o2.float()).abs().max()) <= 8e-3
        assert float((l1 - l2).abs().max()) <= 1e-4


def test_fp8_close_to_unquantised():
    """fp8 Q/K with per-block absmax scales stay close to the unquantised
    result (a check of the quantisation recipe, not of parity)."""
    B, H, S, D = 1, 2, 512, 128
    q8, k8, v, qs, ks = scaled_inputs(B, H, S, S, D, D, 128, 64, "fp8_e4m3", "bf16", seed=79)
    # the same draws before quantisation (Q, then K, from the same seed)
    g = torch.Generator(device="cpu").manual_seed(79)
    q = torch.randn((B, H, S, D), generator=g)
    k = torch.randn((B, H, S, D), generator=g)
    o8, _ = run(q8, k8, v, qs, ks, 128, 64, True)
    o_f, _ = oracle.attn_ref(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                             1 / math.sqrt(D), True)
    err = float(np.max(np.abs(to_np(o8) - o_f)))
    print(f"[fp8 vs unquantised] max|dO|={err:.3e}", flush=True)
    assert err < 0.15


@pytest.mark.parametrize("causal", [True, False])
def test_scaled_fp8_full_size(causal):
    """bf16 V, fp8 Q/K at the long-sequence size (1 x 32 x 16384 x 128), a
    row sample against the oracle."""
    B, H, S, D = 1, 32, 16384, 128
    q, k, v, qs, ks = scaled_inputs(B, H, S, S, D, D, 128, 64, "fp8_e4m3", "bf16", seed=80)
    o, lse = run(q, k, v, qs, ks, 128, 64, causal)
    rows = sample_rows(S, stride=67)   # 67 is coprime with 32: every row position of a wave
    o_s, l_s = to_np(o[:, :, rows]), to_np(lse[:, :, rows])
    del o, lse
    o_ref, lse_ref = ref(q, k, v, qs, ks, 128, 64, causal, rows=rows)
    check(o_s, l_s, o_ref, lse_ref, f"fp8 full size causal={causal} ({len(rows)} rows/slice)")
