"""GPU parity at the largest accepted sizes.

A slice of Q, K, V or O may hold up to 2^31 - 1 bytes (the kernels address
a slice with 32-bit offsets; one byte more is rejected with
TSD_ERR_UNSUPPORTED, see test_abi).  These cases run bf16 slices of just
under 2 GiB, ragged against the tiles, so that the offsets of the last rows
and keys come within a row of 2^31, and check rows at both ends against the
fp64 oracle.  Rows are independent, so the oracle gets only the sampled
query rows (causal rows at or past the last key see every key and are
checked as non-causal ones).
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_scaled_dot_amd as tsd
from tiled_scaled_dot_amd.workloads import random_inputs

pytestmark = pytest.mark.gpu

D = 128
MAX_ROWS = ((1 << 31) - 1) // (D * 2)   # 8388607 bf16 rows of 128 per slice
TOL_O, TOL_LSE = 2e-2, 1e-3


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_rows(o, lse, q, k, v, rows, scale, causal, what):
    rows = sorted(rows)
    o_s, lse_s = to_np(o[:, :, rows]), to_np(lse[:, :, rows])
    kd, vd = k.double().numpy(), v.double().numpy()
    o_ref = np.empty_like(o_s)
    lse_ref = np.empty_like(lse_s)
    S_k = k.shape[2]
    for n, r in enumerate(rows):
        qr = q[:, :, r:r + 1].double().numpy()
        if causal and r < S_k - 1:
            # row r sees keys 0..r: the oracle's causal mask on the first r+1 rows
            qp = q[:, :, :r + 1].double().numpy()
            a, b = oracle.attn_ref(qp, kd, vd, scale, True, rows=[r])
        else:
            a, b = oracle.attn_ref(qr, kd, vd, scale, False)
        o_ref[:, :, n], lse_ref[:, :, n] = a[:, :, 0], b[:, :, 0]
    err_o = float(np.max(np.abs(o_s - o_ref)))
    err_l = float(np.max(np.abs(lse_s - lse_ref)))
    print(f"[parity] {what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert np.isfinite(o_s).all() and np.isfinite(lse_s).all()
    assert err_o <= TOL_O and err_l <= TOL_LSE, what


@pytest.fixture(scope="module")
def long_kv():
    """K and V slices of 2^31 - 256 bytes (8388607 keys): CPU bf16, GPU,
    and float64 for the oracle; with 300 query rows."""
    q, k, v = random_inputs((1, 1, 300, D), (1, 1, MAX_ROWS, D), (1, 1, MAX_ROWS, D), "bf16",
                            seed=31)
    return dict(q=q, k=k, v=v, kg=k.cuda(), vg=v.cuda(), kd=k.double().numpy(),
                vd=v.double().numpy())


def test_longest_key_slice(long_kv):
    q, k, v = long_kv["q"], long_kv["k"], long_kv["v"]
    print(f"[case] bf16 S_q={q.shape[2]} S_k={k.shape[2]} D={D} non-causal", flush=True)
    scale = 1 / np.sqrt(D)
    o, lse = tsd.attn_fwd(q.cuda(), long_kv["kg"], long_kv["vg"], scale=scale, causal=False)
    torch.cuda.synchronize()
    check_rows(o, lse, q, k, v, [0, 1, 255, 256, 298, 299], scale, False, "longest key slice")


def check_ext_rows(o, lse, long_kv, rows, scale, what, **mask):
    o_s, lse_s = to_np(o[:, :, rows]), to_np(lse[:, :, rows])
    o_ref, lse_ref = oracle.attn_ref_ext(long_kv["q"].double().numpy(), long_kv["kd"],
                                         long_kv["vd"], scale, rows=rows, **mask)
    err_o = float(np.max(np.abs(o_s - o_ref)))
    err_l = float(np.max(np.abs(lse_s - lse_ref)))
    print(f"[parity] {what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert np.isfinite(o_s).all() and np.isfinite(lse_s).all()
    assert err_o <= TOL_O and err_l <= TOL_LSE, what


def test_longest_key_slice_window_at_the_end(long_kv):
    """Bottom-right causal with a 3000-key window: every row's keys lie in
    the last 3300 of the slice, so the key tiles start near byte 2^31."""
    q = long_kv["q"]
    S_q, S_k = q.shape[2], MAX_ROWS
    mask = dict(causal=True, causal_offset=S_k - S_q, window=3000)
    print(f"[case] ext bf16 S_q={S_q} S_k={S_k} {mask}", flush=True)
    scale = 1 / np.sqrt(D)
    o, lse = tsd.attn_fwd_ext(q.cuda(), long_kv["kg"], long_kv["vg"], scale=scale, **mask)
    torch.cuda.synchronize()
    check_ext_rows(o, lse, long_kv, [0, 1, 150, 298, 299], scale, "window at the end", **mask)


def test_longest_key_slice_splitkv(long_kv):
    """Split-KV over the whole slice: 16 chunks merged."""
    q = long_kv["q"][:, :, :64].contiguous()
    print(f"[case] split-KV bf16 S_q=64 S_k={MAX_ROWS} 16 chunks", flush=True)
    scale = 1 / np.sqrt(D)
    o, lse = tsd.attn_fwd_splitkv(q.cuda(), long_kv["kg"], long_kv["vg"], scale=scale,
                                  n_splits=16)
    torch.cuda.synchronize()
    check_ext_rows(o, lse, dict(long_kv, q=q), [0, 31, 63], scale, "split-KV 16 chunks",
                   causal=False)


@pytest.mark.parametrize("causal", [False, True])
def test_longest_query_slice(causal):
    """Q and O slices of 2^31 - 256 bytes (8388607 query rows), 100 keys."""
    S_q, S_k = MAX_ROWS, 100
    print(f"[case] bf16 S_q={S_q} S_k={S_k} D={D} causal={causal}", flush=True)
    q, k, v = random_inputs((1, 1, S_q, D), (1, 1, S_k, D), (1, 1, S_k, D), "bf16", seed=32)
    scale = 1 / np.sqrt(D)
    o, lse = tsd.attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal)
    torch.cuda.synchronize()
    rows = [0, 1, 98, 99, 100, S_q // 2, S_q - 257, S_q - 256, S_q - 2, S_q - 1]
    check_rows(o, lse, q, k, v, rows, scale, causal, f"longest query slice causal={causal}")
