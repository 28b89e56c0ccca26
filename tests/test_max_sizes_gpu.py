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


def test_longest_key_slice():
    """K and V slices of 2^31 - 256 bytes (8388607 keys), 300 query rows."""
    S_q, S_k = 300, MAX_ROWS
    print(f"[case] bf16 S_q={S_q} S_k={S_k} D={D} non-causal", flush=True)
    q, k, v = random_inputs((1, 1, S_q, D), (1, 1, S_k, D), (1, 1, S_k, D), "bf16", seed=31)
    scale = 1 / np.sqrt(D)
    o, lse = tsd.attn_fwd(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=False)
    torch.cuda.synchronize()
    check_rows(o, lse, q, k, v, [0, 1, 255, 256, 298, 299], scale, False, "longest key slice")


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
