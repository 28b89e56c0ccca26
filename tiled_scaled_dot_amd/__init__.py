"""MI355X-native (gfx950) tiled scaled-dot-product attention forward.

Thin ctypes binding over ``libtsd_attn.so`` (C ABI in ``include/tsd_attn.h``).
This module only marshals arguments: every step of the computation runs in
the library's HIP kernels.  PyTorch supplies device memory and streams.
There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["attn_fwd", "attn_fwd_plan", "attn_fwd_plan_block", "attn_status_string",
           "attn_fwd_ext", "attn_fwd_partial", "attn_merge", "attn_splitkv_plan",
           "attn_fwd_splitkv", "attn_fwd_splitkv_noalloc", "attn_fwd_scaled", "TsdMask",
           "TsdError", "library", "NOALLOC_SCRATCH_BYTES",
           "LIBRARY_PATH",
           "DTYPE_CODES", "STATUS"]

LIBRARY_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtsd_attn.so")

STATUS = {
    0: "TSD_OK",
    1: "TSD_ERR_NULL",
    2: "TSD_ERR_SHAPE",
    3: "TSD_ERR_UNSUPPORTED",
    4: "TSD_ERR_SCALE",
    5: "TSD_ERR_ALIAS",
    6: "TSD_ERR_HIP",
    7: "TSD_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 64 << 20   # TSD_NOALLOC_SCRATCH_BYTES of the C header
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "fp8_e4m3": 3}

EXPORTED = ("attn_fwd", "attn_fwd_plan", "attn_fwd_plan_block", "attn_status_string",
            "attn_fwd_ext", "attn_fwd_partial", "attn_merge", "attn_splitkv_plan",
            "attn_fwd_splitkv", "attn_fwd_scaled", "attn_fwd_splitkv_noalloc")


class TsdError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"{STATUS.get(status, status)}: {text}")
        self.status = status


class TsdPlan(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("block_m", ctypes.c_int32),
        ("block_n", ctypes.c_int32),
        ("dqk_block", ctypes.c_int32),
        ("dv_block", ctypes.c_int32),
        ("waves", ctypes.c_int32),
        ("threads", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32),
        ("order", ctypes.c_int32),
        ("slices", ctypes.c_int64),
        ("q_blocks", ctypes.c_int64),
        ("kv_blocks", ctypes.c_int64),
        ("grid", ctypes.c_int64),
        ("total_kv_steps", ctypes.c_int64),
        ("vector_io", ctypes.c_int64),
        ("key_split", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class TsdMask(ctypes.Structure):
    """Key visibility of the extended entry points: row i sees keys
    [max(kv_begin, i + causal_offset - window + 1) if window else kv_begin,
     min(kv_end, i + causal_offset + 1) if causal else kv_end)."""
    _fields_ = [
        ("causal_offset", ctypes.c_int64),
        ("window", ctypes.c_int64),
        ("kv_begin", ctypes.c_int64),
        ("kv_end", ctypes.c_int64),
    ]


def make_mask(S_k, causal_offset=0, window=0, kv_begin=0, kv_end=None) -> TsdMask:
    return TsdMask(int(causal_offset), int(window), int(kv_begin),
                   int(S_k if kv_end is None else kv_end))


_lib = None


def library(path: str = LIBRARY_PATH) -> ctypes.CDLL:
    """Load libtsd_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m tiled_scaled_dot_amd.build` (there is no fallback)")
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                             ctypes.c_float, ctypes.c_int, ctypes.c_int, vp]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_plan.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                                  ctypes.POINTER(TsdPlan)]
    lib.attn_fwd_plan.restype = ctypes.c_int
    lib.attn_fwd_plan_block.argtypes = [ctypes.POINTER(TsdPlan), i64, i64, i64,
                                        ctypes.POINTER(i64), ctypes.POINTER(i64),
                                        ctypes.POINTER(i64)]
    lib.attn_fwd_plan_block.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    mp, f, ci = ctypes.POINTER(TsdMask), ctypes.c_float, ctypes.c_int
    lib.attn_fwd_ext.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, f, ci,
                                 ci, mp, vp]
    lib.attn_fwd_ext.restype = ci
    lib.attn_fwd_partial.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, f,
                                     ci, ci, mp, i64, i64, vp]
    lib.attn_fwd_partial.restype = ci
    lib.attn_merge.argtypes = [vp, vp, i64, i64, i64, i64, i64, vp, vp, ci, vp]
    lib.attn_merge.restype = ci
    lib.attn_splitkv_plan.argtypes = [i64, i64, i64, i64, i64, i64, i64, ci, ci, mp, i64,
                                      ctypes.POINTER(i64), ctypes.POINTER(i64),
                                      ctypes.POINTER(i64)]
    lib.attn_splitkv_plan.restype = ci
    lib.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, f,
                                     ci, ci, mp, i64, vp, i64, vp]
    lib.attn_fwd_splitkv.restype = ci
    lib.attn_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                             i64, f, ci, ci, mp, i64, vp]
    lib.attn_fwd_splitkv_noalloc.restype = ci
    lib.attn_fwd_scaled.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                    i64, i64, ci, ci, ci, vp]
    lib.attn_fwd_scaled.restype = ci
    _lib = lib
    return lib


def attn_status_string(status: int) -> str:
    return library().attn_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise TsdError(status, attn_status_string(status))


def attn_fwd_plan(B, H, S_q, S_k, D_qk, D_v, causal=False, dtype="bf16") -> TsdPlan:
    plan = TsdPlan()
    code = DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    _check(library().attn_fwd_plan(B, H, S_q, S_k, D_qk, D_v, int(bool(causal)), code,
                                   ctypes.byref(plan)))
    return plan


def attn_fwd_plan_block(plan: TsdPlan, S_q: int, S_k: int, block: int):
    """(query block, slice, key tiles visited) of workgroup `block`."""
    qb, sl, steps = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(library().attn_fwd_plan_block(ctypes.byref(plan), S_q, S_k, block, ctypes.byref(qb),
                                         ctypes.byref(sl), ctypes.byref(steps)))
    return qb.value, sl.value, steps.value


def attn_fwd_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S_q, S_k, D_qk, D_v, scale,
                 causal, dtype, stream=None) -> int:
    """Direct call with integer device addresses; returns the TSD status."""
    code = DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    return library().attn_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, S_q, S_k, D_qk, D_v,
                              float(scale), int(bool(causal)), code, stream)


def _code(dtype) -> int:
    return DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)


def _mask_ref(mask):
    return None if mask is None else ctypes.byref(mask)


def attn_fwd_ext_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, H_kv, S_q, S_k, D_qk, D_v,
                     scale, causal, dtype, mask=None, stream=None) -> int:
    return library().attn_fwd_ext(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, H_kv, S_q, S_k,
                                  D_qk, D_v, float(scale), int(bool(causal)), _code(dtype),
                                  _mask_ref(mask), stream)


def attn_fwd_partial_raw(q_ptr, k_ptr, v_ptr, op_ptr, lp_ptr, B, H, H_kv, S_q, S_k, D_qk,
                         D_v, scale, causal, dtype, mask, n_splits, split_len,
                         stream=None) -> int:
    return library().attn_fwd_partial(q_ptr, k_ptr, v_ptr, op_ptr, lp_ptr, B, H, H_kv, S_q,
                                      S_k, D_qk, D_v, float(scale), int(bool(causal)),
                                      _code(dtype), _mask_ref(mask), n_splits, split_len,
                                      stream)


def attn_merge_raw(op_ptr, lp_ptr, n_parts, B, H, S_q, D_v, o_ptr, lse_ptr, dtype,
                   stream=None) -> int:
    return library().attn_merge(op_ptr, lp_ptr, n_parts, B, H, S_q, D_v, o_ptr, lse_ptr,
                                _code(dtype), stream)


def attn_fwd_splitkv_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, H_kv, S_q, S_k, D_qk,
                         D_v, scale, causal, dtype, mask, n_splits, ws_ptr, ws_bytes,
                         stream=None) -> int:
    return library().attn_fwd_splitkv(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, H_kv, S_q,
                                      S_k, D_qk, D_v, float(scale), int(bool(causal)),
                                      _code(dtype), _mask_ref(mask), n_splits, ws_ptr,
                                      ws_bytes, stream)


def attn_splitkv_plan(B, H, S_q, S_k, D_qk, D_v, causal=False, dtype="bf16", mask=None,
                      n_splits=0, H_kv=None):
    """(chunks, keys per chunk, workspace bytes) attn_fwd_splitkv would use."""
    n, ln, ws = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(library().attn_splitkv_plan(B, H, H if H_kv is None else H_kv, S_q, S_k, D_qk, D_v,
                                       int(bool(causal)), _code(dtype), _mask_ref(mask),
                                       n_splits, ctypes.byref(n), ctypes.byref(ln),
                                       ctypes.byref(ws)))
    return n.value, ln.value, ws.value


def _qkv(q, k, v, grouped=False):
    """Validate q, k, v tensors; returns (dtype code, B, H, S_q, S_k, D_qk, D_v)
    (with H_kv appended when ``grouped``: k and v may then hold fewer heads,
    a divisor of q's)."""
    import torch

    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if q.dtype not in codes or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype among float32, float16, bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B,H,S,D]")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _one_device(q, k=k, v=v)
    B, H, S_q, D_qk = q.shape
    S_k, D_v = k.shape[2], v.shape[3]
    H_kv = k.shape[1] if grouped else H
    if (tuple(k.shape) != (B, H_kv, S_k, D_qk) or tuple(v.shape) != (B, H_kv, S_k, D_v)
            or H % H_kv != 0):
        raise ValueError(f"inconsistent shapes q{tuple(q.shape)} k{tuple(k.shape)} "
                         f"v{tuple(v.shape)}")
    if grouped:
        return codes[q.dtype], B, H, H_kv, S_q, S_k, D_qk, D_v
    return codes[q.dtype], B, H, S_q, S_k, D_qk, D_v


def _buffer(t, shape, dtype, like, name):
    import torch

    if t is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    if (tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous()
            or t.device != like.device):
        raise ValueError(f"{name} must be a contiguous {dtype} {list(shape)} tensor on "
                         f"{like.device}")
    return t


def _stream(stream, device):
    import torch

    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _one_device(first, **others):
    """Every tensor of a call must live on the first one's device."""
    for name, t in others.items():
        if t is not None and t.device != first.device:
            raise ValueError(f"{name} is on {t.device}, the call's tensors on {first.device}")


def _on(t):
    """Make t's device the current one for the call: the library launches on
    the current device, into a stream of that device."""
    import torch

    return torch.cuda.device(t.device)


def attn_fwd_ext(q, k, v, scale=None, causal=False, causal_offset=0, window=0, kv_begin=0,
                 kv_end=None, out=None, lse=None, stream=None):
    """attn_fwd restricted per row to the keys of the mask (see TsdMask);
    rows that see no key get O = 0 and LSE = -inf.  16-bit inputs only.  k
    and v may hold H_kv heads (a divisor of q's H): head h reads K/V head
    h // (H // H_kv)."""
    import torch

    code, B, H, H_kv, S_q, S_k, D_qk, D_v = _qkv(q, k, v, grouped=True)
    if scale is None:
        scale = 1.0 / math.sqrt(D_qk)
    out = _buffer(out, (B, H, S_q, D_v), q.dtype, q, "out")
    lse = _buffer(lse, (B, H, S_q), torch.float32, q, "lse")
    mask = make_mask(S_k, causal_offset, window, kv_begin, kv_end)
    with _on(q):
        _check(attn_fwd_ext_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), B, H, H_kv, S_q, S_k, D_qk, D_v, scale, causal,
                                code, mask, _stream(stream, q.device)))
    return out, lse


def attn_fwd_partial(q, k, v, n_splits, split_len, scale=None, causal=False, causal_offset=0,
                     window=0, kv_begin=0, kv_end=None, o_parts=None, lse_parts=None,
                     stream=None):
    """Per-chunk partial results: O_parts [n,B,H,S_q,D_v] and LSE_parts
    [n,B,H,S_q], both float32; chunk s covers keys kv_begin + s*split_len
    onwards (split_len keys, cut to the range)."""
    import torch

    code, B, H, H_kv, S_q, S_k, D_qk, D_v = _qkv(q, k, v, grouped=True)
    if scale is None:
        scale = 1.0 / math.sqrt(D_qk)
    o_parts = _buffer(o_parts, (n_splits, B, H, S_q, D_v), torch.float32, q, "o_parts")
    lse_parts = _buffer(lse_parts, (n_splits, B, H, S_q), torch.float32, q, "lse_parts")
    mask = make_mask(S_k, causal_offset, window, kv_begin, kv_end)
    with _on(q):
        _check(attn_fwd_partial_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_parts.data_ptr(),
                                    lse_parts.data_ptr(), B, H, H_kv, S_q, S_k, D_qk, D_v, scale,
                                    causal, code, mask, n_splits, split_len,
                                    _stream(stream, q.device)))
    return o_parts, lse_parts


def attn_merge(o_parts, lse_parts, dtype=None, out=None, lse=None, stream=None):
    """Merge partial results: o_parts [n,B,H,S_q,D_v], lse_parts [n,B,H,S_q]
    (float32) -> O [B,H,S_q,D_v] (``dtype``, default float32), LSE [B,H,S_q]."""
    import torch

    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    dtype = torch.float32 if dtype is None else dtype
    if o_parts.dim() != 5 or lse_parts.dim() != 4:
        raise ValueError("o_parts must be [n,B,H,S_q,D_v] and lse_parts [n,B,H,S_q]")
    n, B, H, S_q, D_v = o_parts.shape
    for name, t in (("o_parts", o_parts), ("lse_parts", lse_parts)):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 GPU tensor")
    if tuple(lse_parts.shape) != (n, B, H, S_q):
        raise ValueError("lse_parts shape does not match o_parts")
    _one_device(o_parts, lse_parts=lse_parts)
    out = _buffer(out, (B, H, S_q, D_v), dtype, o_parts, "out")
    lse = _buffer(lse, (B, H, S_q), torch.float32, o_parts, "lse")
    with _on(o_parts):
        _check(attn_merge_raw(o_parts.data_ptr(), lse_parts.data_ptr(), n, B, H, S_q, D_v,
                              out.data_ptr(), lse.data_ptr(), codes[dtype],
                              _stream(stream, o_parts.device)))
    return out, lse


def attn_fwd_splitkv(q, k, v, scale=None, causal=False, causal_offset=0, window=0, kv_begin=0,
                     kv_end=None, n_splits=0, workspace=None, out=None, lse=None, stream=None):
    """attn_fwd_ext computed over key chunks and merged (n_splits <= 0: the
    library's choice).  ``workspace``: a uint8 GPU tensor of at least the
    planned size (allocated here when None)."""
    import torch

    code, B, H, H_kv, S_q, S_k, D_qk, D_v = _qkv(q, k, v, grouped=True)
    if scale is None:
        scale = 1.0 / math.sqrt(D_qk)
    out = _buffer(out, (B, H, S_q, D_v), q.dtype, q, "out")
    lse = _buffer(lse, (B, H, S_q), torch.float32, q, "lse")
    mask = make_mask(S_k, causal_offset, window, kv_begin, kv_end)
    _, _, ws = attn_splitkv_plan(B, H, S_q, S_k, D_qk, D_v, causal, code, mask, n_splits,
                                 H_kv=H_kv)
    if workspace is None and ws > 0:
        workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
    _one_device(q, workspace=workspace)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with _on(q):
        _check(attn_fwd_splitkv_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), B, H, H_kv, S_q, S_k, D_qk, D_v, scale, causal,
                                    code, mask, n_splits, ws_ptr, ws_bytes,
                                    _stream(stream, q.device)))
    return out, lse


def attn_fwd_splitkv_noalloc_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, H_kv, S_q, S_k,
                                 D_qk, D_v, scale, causal, dtype, mask, n_splits,
                                 stream=None) -> int:
    return library().attn_fwd_splitkv_noalloc(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, H_kv,
                                              S_q, S_k, D_qk, D_v, float(scale),
                                              int(bool(causal)), _code(dtype), _mask_ref(mask),
                                              n_splits, stream)


def attn_fwd_splitkv_noalloc(q, k, v, scale=None, causal=False, causal_offset=0, window=0,
                             kv_begin=0, kv_end=None, n_splits=0, out=None, lse=None,
                             stream=None):
    """attn_fwd_splitkv with the partial results in the library's fixed
    per-device scratch array (NOALLOC_SCRATCH_BYTES): the library allocates
    nothing.  Pass ``out`` and ``lse`` to allocate nothing here either.
    Calls that overlap on one GPU share the array and race."""
    import torch

    code, B, H, H_kv, S_q, S_k, D_qk, D_v = _qkv(q, k, v, grouped=True)
    if scale is None:
        scale = 1.0 / math.sqrt(D_qk)
    out = _buffer(out, (B, H, S_q, D_v), q.dtype, q, "out")
    lse = _buffer(lse, (B, H, S_q), torch.float32, q, "lse")
    mask = make_mask(S_k, causal_offset, window, kv_begin, kv_end)
    with _on(q):
        _check(attn_fwd_splitkv_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                            out.data_ptr(), lse.data_ptr(), B, H, H_kv, S_q, S_k,
                                            D_qk, D_v, scale, causal, code, mask, n_splits,
                                            _stream(stream, q.device)))
    return out, lse


def attn_fwd_scaled_raw(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, qs_ptr, ks_ptr, B, H, S_q, S_k,
                        D_qk, D_v, q_block, k_block, causal, qk_dtype, dtype,
                        stream=None) -> int:
    return library().attn_fwd_scaled(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, qs_ptr, ks_ptr, B, H,
                                     S_q, S_k, D_qk, D_v, q_block, k_block, int(bool(causal)),
                                     _code(qk_dtype), _code(dtype), stream)


def attn_fwd_scaled(q, k, v, q_scale, k_scale, q_block, k_block, causal=False, out=None,
                    lse=None, stream=None):
    """Base-2 attention with per-block scales: score = q_scale[b,h,i//q_block]
    * k_scale[b,h,j//k_block] * (q_i . k_j), weights 2^score.  q, k:
    float8_e4m3fn, or v's dtype (float16 / bfloat16); q_scale, k_scale:
    float32 [B,H,ceil(S/block)], finite, of either sign; k_block a multiple
    of 64.
    Returns O (v's dtype) and LSE (float32, natural log)."""
    import torch

    vcodes = {torch.float16: 1, torch.bfloat16: 2}
    if v.dtype not in vcodes:
        raise TypeError("v must be float16 or bfloat16")
    qk_code = 3 if q.dtype == torch.float8_e4m3fn else vcodes.get(q.dtype)
    if qk_code is None or k.dtype != q.dtype or (qk_code != 3 and q.dtype != v.dtype):
        raise TypeError("q and k must be float8_e4m3fn, or v's dtype")
    for name, t in (("q", q), ("k", k), ("v", v), ("q_scale", q_scale), ("k_scale", k_scale)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    _one_device(v, q=q, k=k, q_scale=q_scale, k_scale=k_scale)
    B, H, S_q, D_qk = q.shape
    S_k, D_v = k.shape[2], v.shape[3]
    if tuple(k.shape) != (B, H, S_k, D_qk) or tuple(v.shape) != (B, H, S_k, D_v):
        raise ValueError("inconsistent q/k/v shapes")
    nq, nk = -(-S_q // q_block), -(-S_k // k_block)
    if (tuple(q_scale.shape) != (B, H, nq) or tuple(k_scale.shape) != (B, H, nk)
            or q_scale.dtype != torch.float32 or k_scale.dtype != torch.float32):
        raise ValueError(f"q_scale must be float32 [{B},{H},{nq}] and k_scale [{B},{H},{nk}]")
    out = _buffer(out, (B, H, S_q, D_v), v.dtype, v, "out")
    lse = _buffer(lse, (B, H, S_q), torch.float32, v, "lse")
    with _on(v):
        _check(attn_fwd_scaled_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), q_scale.data_ptr(), k_scale.data_ptr(), B, H,
                                   S_q, S_k, D_qk, D_v, q_block, k_block, causal, qk_code,
                                   vcodes[v.dtype], _stream(stream, v.device)))
    return out, lse


def attn_fwd(q, k, v, scale=None, causal=False, out=None, lse=None, stream=None):
    """O, LSE = softmax(q k^T * scale) v  (per batch and head).

    q [B,H,S_q,D_qk], k [B,H,S_k,D_qk], v [B,H,S_k,D_v]: contiguous CUDA
    tensors of one dtype (float32, float16 or bfloat16).  ``scale`` defaults
    to 1/sqrt(D_qk).  Returns O [B,H,S_q,D_v] (input dtype) and LSE
    [B,H,S_q] (float32).  Runs on ``stream`` (default: torch's current
    stream) and does not synchronise.
    """
    import torch

    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if q.dtype not in codes or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype among float32, float16, bfloat16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B,H,S,D]")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _one_device(q, k=k, v=v)
    B, H, S_q, D_qk = q.shape
    S_k, D_v = k.shape[2], v.shape[3]
    if tuple(k.shape) != (B, H, S_k, D_qk) or tuple(v.shape) != (B, H, S_k, D_v):
        raise ValueError(f"inconsistent shapes q{tuple(q.shape)} k{tuple(k.shape)} "
                         f"v{tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D_qk)
    if out is None:
        out = torch.empty((B, H, S_q, D_v), dtype=q.dtype, device=q.device)
    elif (tuple(out.shape) != (B, H, S_q, D_v) or out.dtype != q.dtype
          or not out.is_contiguous() or out.device != q.device):
        raise ValueError("out must be a contiguous [B,H,S_q,D_v] tensor like q")
    if lse is None:
        lse = torch.empty((B, H, S_q), dtype=torch.float32, device=q.device)
    elif (tuple(lse.shape) != (B, H, S_q) or lse.dtype != torch.float32
          or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B,H,S_q] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    with _on(q):
        status = attn_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), B, H, S_q, S_k, D_qk, D_v, scale, causal,
                              codes[q.dtype], stream)
    _check(status)
    return out, lse
