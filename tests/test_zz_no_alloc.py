"""attn_fwd_splitkv_noalloc (the split-KV entry point that stages its
partial results in the library's fixed per-device scratch array) against
attn_fwd_splitkv with a caller workspace, through the C ABI: two calls in a
row, the second smaller, each bitwise equal to the workspace path and
within the 16-bit parity bar of the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_scaled_dot_amd as tsd
from tiled_scaled_dot_amd.workloads import random_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run_pair(shape, dtype, causal, coff, window, n_splits, seed):
    B, H, H_kv, S_q, S_k, D_qk, D_v = shape
    q, k, v = random_inputs((B, H, S_q, D_qk), (B, H_kv, S_k, D_qk), (B, H_kv, S_k, D_v),
                            dtype, seed=seed)
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    scale = 1.0 / math.sqrt(D_qk)
    mask = tsd.make_mask(S_k, coff, window)
    n, _, ws = tsd.attn_splitkv_plan(B, H, S_q, S_k, D_qk, D_v, causal, dtype, mask, n_splits,
                                     H_kv=H_kv)
    assert n > 1 and 0 < ws <= tsd.NOALLOC_SCRATCH_BYTES
    print(f"[case] noalloc {shape} {dtype} causal={causal} chunks={n} scratch={ws}",
          flush=True)
    # outputs poisoned with NaN: every element must be written
    o1 = torch.full((B, H, S_q, D_v), float("nan"), dtype=qg.dtype, device=DEV)
    l1 = torch.full((B, H, S_q), float("nan"), dtype=torch.float32, device=DEV)
    st = tsd.attn_fwd_splitkv_noalloc_raw(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(),
                                          o1.data_ptr(), l1.data_ptr(), B, H, H_kv, S_q, S_k,
                                          D_qk, D_v, scale, causal, dtype, mask, n_splits,
                                          torch.cuda.current_stream().cuda_stream)
    assert st == 0, tsd.attn_status_string(st)
    o2, l2 = tsd.attn_fwd_splitkv(qg, kg, vg, scale=scale, causal=causal, causal_offset=coff,
                                  window=window, n_splits=n_splits)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "differs from the workspace path"
    o_ref, l_ref = oracle.attn_ref_ext(q.double().numpy(), k.double().numpy(),
                                       v.double().numpy(), scale, causal, causal_offset=coff,
                                       window=window)
    err_o = float(np.max(np.abs(o1.float().cpu().numpy() - o_ref)))
    err_l = float(np.max(np.abs(l1.cpu().numpy() - l_ref)))
    print(f"[parity] noalloc: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= 2e-2 and err_l <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_noalloc_two_calls_second_smaller(dtype):
    # a long-context prefill shape, then a smaller grouped-head decode shape
    # on the same scratch array
    _run_pair((1, 4, 4, 256, 9000, 128, 128), dtype, True, 9000 - 256, 0, 8, seed=11)
    _run_pair((2, 8, 2, 1, 3000, 64, 128), dtype, True, 3000 - 1, 0, 5, seed=12)


def test_noalloc_single_chunk_and_oversized():
    # one chunk: no scratch at all; result equals attn_fwd_ext
    q, k, v = random_inputs((1, 2, 200, 64), (1, 2, 300, 64), (1, 2, 300, 64), "bf16", seed=13)
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    o1, l1 = tsd.attn_fwd_splitkv_noalloc(qg, kg, vg, causal=True, n_splits=1)
    o2, l2 = tsd.attn_fwd_ext(qg, kg, vg, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # partial results beyond the array: TSD_ERR_SCRATCH, nothing written
    B, H, S_q, S_k, D = 1, 16, 2048, 4096, 128
    n, _, ws = tsd.attn_splitkv_plan(B, H, S_q, S_k, D, D, False, "bf16", None, 8)
    assert ws > tsd.NOALLOC_SCRATCH_BYTES
    qb = torch.zeros((B, H, S_q, D), dtype=torch.bfloat16, device=DEV)
    kb = torch.zeros((B, H, S_k, D), dtype=torch.bfloat16, device=DEV)
    out = torch.full((B, H, S_q, D), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tsd.TsdError) as e:
        tsd.attn_fwd_splitkv_noalloc(qb, kb, kb, n_splits=8, out=out)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
