"""Seeded random configurations across the entry points, each against the
fp64 oracle (the same bars as the targeted tests).  Most shapes are drawn
so that the oracle checks every output (a few million score elements at
most) while covering ragged sizes, head-dim tails, D_qk != D_v, both 16-bit
dtypes, causal offsets, windows, key ranges, grouped heads and chunk
counts; a last group draws grids of up to 6000 x 6000 per slice and checks
a row sample.

TSD_RANDOM_SEEDS=N in the environment widens every group to at least N
seeds (a longer sweep of the same generators; the default keeps the suite
short)."""
import math
import os
import random

import numpy as np
import pytest
import torch

import oracle
import tiled_scaled_dot_amd as tsd
from tiled_scaled_dot_amd.workloads import random_inputs, scaled_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL_O = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}
TOL_LSE = {"f32": 1e-4, "f16": 1e-3, "bf16": 1e-3}
N_SEEDS = int(os.environ.get("TSD_RANDOM_SEEDS", "0"))


def seeds(default):
    return range(max(default, N_SEEDS))


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(o, lse, o_ref, lse_ref, dtype, what):
    o, lse = to_np(o), to_np(lse)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty rows differ"
    assert np.all(o[empty] == 0.0), f"{what}: empty row with nonzero O"
    live = ~empty
    if live.any():
        err_o = float(np.max(np.abs(o[live] - o_ref[live])))
        err_l = float(np.max(np.abs(lse[live] - lse_ref[live])))
        assert err_o <= TOL_O[dtype] and err_l <= TOL_LSE[dtype], \
            f"{what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}"


def draw_plain(rng):
    dtype = rng.choice(["f32", "f16", "bf16"])
    return dict(dtype=dtype, B=rng.randint(1, 2), H=rng.randint(1, 4), S_q=rng.randint(1, 700),
                S_k=rng.randint(1, 900), D_qk=rng.randint(1, 128), D_v=rng.randint(1, 128),
                causal=rng.random() < 0.5, scale=rng.uniform(-0.3, 0.3))


def draw_ext(rng):
    dtype = rng.choice(["f16", "bf16"])
    H_kv = rng.choice([1, 2, 4])
    S_k = rng.randint(1, 1500)
    kb = rng.randint(0, S_k)
    ke = rng.randint(kb, S_k)
    return dict(dtype=dtype, B=rng.randint(1, 2), H=H_kv * rng.choice([1, 2, 3]), H_kv=H_kv,
                S_q=rng.randint(1, 500), S_k=S_k, D_qk=8 * rng.randint(1, 16),
                D_v=8 * rng.randint(1, 16), causal=rng.random() < 0.7,
                coff=rng.randint(-300, 1500), window=rng.choice([0, 0, 1, 37, 300]),
                kv_begin=kb if rng.random() < 0.3 else 0,
                kv_end=ke if rng.random() < 0.3 else None,
                n_splits=rng.choice([1, 1, 2, 3, 7]))


@pytest.mark.parametrize("seed", seeds(12))
def test_random_plain(seed):
    rng = random.Random(1000 + seed)
    c = draw_plain(rng)
    print(f"[case] plain {c}", flush=True)
    q, k, v = random_inputs((c["B"], c["H"], c["S_q"], c["D_qk"]), (c["B"], c["H"], c["S_k"], c["D_qk"]),
                            (c["B"], c["H"], c["S_k"], c["D_v"]), c["dtype"], seed=seed)
    o, lse = tsd.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=c["scale"], causal=c["causal"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_ref(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                     c["scale"], c["causal"])
    check(o, lse, o_ref, lse_ref, c["dtype"], f"plain {c}")


@pytest.mark.parametrize("seed", seeds(16))
def test_random_extended(seed):
    rng = random.Random(2000 + seed)
    c = draw_ext(rng)
    print(f"[case] ext {c}", flush=True)
    B, H, H_kv = c["B"], c["H"], c["H_kv"]
    q, k, v = random_inputs((B, H, c["S_q"], c["D_qk"]), (B, H_kv, c["S_k"], c["D_qk"]),
                            (B, H_kv, c["S_k"], c["D_v"]), c["dtype"], seed=seed)
    scale = 1 / math.sqrt(c["D_qk"])
    kw = dict(scale=scale, causal=c["causal"], causal_offset=c["coff"], window=c["window"],
              kv_begin=c["kv_begin"], kv_end=c["kv_end"])
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    if c["n_splits"] == 1:
        o, lse = tsd.attn_fwd_ext(qg, kg, vg, **kw)
    else:
        o, lse = tsd.attn_fwd_splitkv(qg, kg, vg, n_splits=c["n_splits"], **kw)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_ref_ext(q.double().numpy(), k.double().numpy(),
                                         v.double().numpy(), scale, c["causal"],
                                         causal_offset=c["coff"], window=c["window"],
                                         kv_begin=c["kv_begin"], kv_end=c["kv_end"])
    check(o, lse, o_ref, lse_ref, c["dtype"], f"ext {c}")


@pytest.mark.parametrize("seed", seeds(12))
def test_random_scaled(seed):
    rng = random.Random(3000 + seed)
    qk = rng.choice(["fp8_e4m3", "bf16", "f16"])
    vdt = "f16" if qk == "f16" else "bf16"
    D_qk = rng.choice([128, 112, 96, 80]) if qk == "fp8_e4m3" else 8 * rng.randint(1, 16)
    D_v = rng.choice([64, 128]) if qk == "fp8_e4m3" else 8 * rng.randint(1, 16)
    c = dict(qk=qk, B=1, H=rng.randint(1, 3), S_q=rng.randint(1, 600), S_k=rng.randint(1, 900),
             D_qk=D_qk, D_v=D_v, q_block=rng.choice([1, 16, 128, 300]),
             k_block=64 * rng.randint(1, 4), causal=rng.random() < 0.5)
    print(f"[case] scaled {c}", flush=True)
    q, k, v, qs, ks = scaled_inputs(c["B"], c["H"], c["S_q"], c["S_k"], c["D_qk"], c["D_v"],
                                    c["q_block"], c["k_block"], qk, vdt, seed=seed,
                                    scale_jitter=True)
    # block scales of either sign (and some zero), drawn per block
    g = torch.Generator(device="cpu").manual_seed(3100 + seed)
    ks = (ks * torch.randint(-1, 2, ks.shape, generator=g).float()).contiguous()
    qs = (qs * torch.where(torch.rand(qs.shape, generator=g) < 0.25, -1.0, 1.0)).contiguous()
    o, lse = tsd.attn_fwd_scaled(q.to(DEV), k.to(DEV), v.to(DEV), qs.to(DEV), ks.to(DEV),
                                 c["q_block"], c["k_block"], c["causal"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attn_ref_scaled(q.double().numpy(), k.double().numpy(),
                                            v.double().numpy(), qs.double().numpy(),
                                            ks.double().numpy(), c["q_block"], c["k_block"],
                                            c["causal"])
    check(o, lse, o_ref, lse_ref, vdt, f"scaled {c}")


def draw_large(rng):
    dtype = rng.choice(["f16", "bf16", "bf16", "f32"])
    D_qk = rng.choice([64, 128, rng.randint(1, 128)])
    return dict(dtype=dtype, B=rng.randint(1, 2), H=rng.randint(1, 6), S_q=rng.randint(1, 6000),
                S_k=rng.randint(1, 6000), D_qk=D_qk, D_v=rng.choice([64, 128, rng.randint(1, 128)]),
                causal=rng.random() < 0.5,
                scale=rng.choice([1 / math.sqrt(D_qk), rng.uniform(-0.4, 0.4)]))


@pytest.mark.parametrize("seed", seeds(10))
def test_random_large_sampled_rows(seed):
    """Grids of up to a few thousand rows and keys (many key tiles, several
    workgroups per CU), every output computed on the GPU and a random sample
    of rows, plus the first and last, checked exactly against the oracle."""
    rng = random.Random(4000 + seed)
    c = draw_large(rng)
    print(f"[case] large {c}", flush=True)
    q, k, v = random_inputs((c["B"], c["H"], c["S_q"], c["D_qk"]), (c["B"], c["H"], c["S_k"], c["D_qk"]),
                            (c["B"], c["H"], c["S_k"], c["D_v"]), c["dtype"], seed=4000 + seed)
    o, lse = tsd.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=c["scale"], causal=c["causal"])
    torch.cuda.synchronize()
    rows = sorted({0, c["S_q"] - 1} | {rng.randrange(c["S_q"]) for _ in range(48)})
    o_ref, lse_ref = oracle.attn_ref(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                     c["scale"], c["causal"], rows=rows)
    check(o[:, :, rows], lse[:, :, rows], o_ref, lse_ref, c["dtype"], f"large {c}")
