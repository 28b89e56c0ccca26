"""Host-side checks of the C ABI (no GPU needed).

* the library loads and exports every function include/tsd_attn.h declares;
* every invalid call returns its status before any HIP call (fake device
  addresses are never dereferenced because nothing is launched);
* the planner: grid, key-tile counts, causal work, heaviest-first order,
  XCD grouping, and exactly-once coverage of every (query block, slice).
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

import tiled_scaled_dot_amd as tsd
from tiled_scaled_dot_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsd_attn.h")

pytestmark = pytest.mark.cpu


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tsd.LIBRARY_PATH):
        from tiled_scaled_dot_amd import build
        build.build()
    return tsd.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(tsd.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", tsd.LIBRARY_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, f"{name} not exported"
    # nothing else: the internals are built with hidden visibility
    assert exported == set(declared_functions()), sorted(exported - set(declared_functions()))


def test_status_strings(lib):
    for code in range(8):
        assert tsd.attn_status_string(code)
    assert tsd.attn_status_string(99) == "unknown status"


# Fake, 256-byte aligned, non-overlapping device addresses: every call below
# must be rejected on the host, so none is ever dereferenced.
QA, KA, VA, OA, LA = (0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000)
GOOD = dict(B=1, H=2, S_q=128, S_k=128, D_qk=64, D_v=64)


def call(q=QA, k=KA, v=VA, o=OA, lse=LA, scale=0.125, causal=0, dtype=2, **dims):
    d = dict(GOOD)
    d.update(dims)
    return tsd.attn_fwd_raw(q, k, v, o, lse, d["B"], d["H"], d["S_q"], d["S_k"], d["D_qk"],
                            d["D_v"], scale, causal, dtype)


@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_null_pointer(lib, which):
    assert call(**{which: None}) == 1


@pytest.mark.parametrize("dim", ["B", "H", "S_q", "S_k", "D_qk", "D_v"])
@pytest.mark.parametrize("value", [0, -1])
def test_bad_shape(lib, dim, value):
    assert call(**{dim: value}) == 2


@pytest.mark.parametrize("dims", [dict(D_qk=129), dict(D_v=129), dict(D_qk=256, D_v=256)])
def test_head_dim_above_block_width(lib, dims):
    assert call(**dims) == 3


@pytest.mark.parametrize("dtype", [-1, 3, 7])
def test_unknown_dtype(lib, dtype):
    assert call(dtype=dtype) == 3


def test_slice_too_large(lib):
    # a single slice of 2^31 bytes or more is rejected (32-bit in-slice offsets)
    assert call(S_q=(1 << 24), D_qk=128, dtype=0) == 3
    assert call(S_k=(1 << 24), D_v=128, dtype=0) == 3


def test_misaligned(lib):
    assert call(q=QA + 1) == 3          # not element aligned (bf16)
    assert call(o=OA + 2, dtype=0) == 3  # not element aligned (f32)
    assert call(lse=LA + 2) == 3


@pytest.mark.parametrize("scale", [float("nan"), float("inf"), float("-inf")])
def test_scale_not_finite(lib, scale):
    assert call(scale=scale) == 4


@pytest.mark.parametrize("o,lse", [(QA, LA), (KA + 64, LA), (VA - 4096, LA),
                                   (OA, QA + 8), (OA, OA + 100), (OA, VA)])
def test_aliasing(lib, o, lse):
    assert call(o=o, lse=lse) == 5


def test_output_adjacent_is_not_alias(lib):
    # O ends exactly where LSE begins: no overlap, so the call passes validation
    # and would launch; only the plan is checked here.
    o_bytes = 1 * 2 * 128 * 64 * 2
    plan = tsd.attn_fwd_plan(1, 2, 128, 128, 64, 64, False, "bf16")
    assert plan.grid == 2
    assert OA + o_bytes <= LA


def test_plan_errors(lib):
    with pytest.raises(tsd.TsdError) as e:
        tsd.attn_fwd_plan(1, 1, 0, 4, 64, 64)
    assert e.value.status == 2
    with pytest.raises(tsd.TsdError) as e:
        tsd.attn_fwd_plan(1, 1, 4, 4, 200, 64)
    assert e.value.status == 3
    assert lib.attn_fwd_plan(1, 1, 4, 4, 8, 8, 0, 2, None) == 1


# ------------------------------------------------------------------ planner
def expected_tiles(qb, bm, bn, S_q, S_k, causal):
    if not causal:
        return math.ceil(S_k / bn)
    last_q = min((qb + 1) * bm, S_q) - 1
    return math.ceil(min(last_q + 1, S_k) / bn)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_plan_for_workloads(lib, name):
    w = WORKLOADS[name]
    plan = tsd.attn_fwd_plan(w.B, w.H, w.S_q, w.S_k, w.D_qk, w.D_v, w.causal, w.dtype)
    if w.dtype == "f32" and plan.key_split > 1:
        # f32 on a small grid: 32 rows per workgroup, the 4 waves split the
        # 32-key tiles (one LDS region each, combined at the end)
        assert (plan.block_m, plan.threads, plan.waves, plan.block_n) == (32, 256, 4, 32)
        assert plan.key_split == 4
        assert plan.lds_bytes <= 160 * 1024
    elif w.dtype == "f32":
        # generic kernel: 4 waves x 32 rows, 32-key tiles, two LDS stages
        assert (plan.block_m, plan.threads, plan.waves, plan.block_n) == (128, 256, 4, 32)
        assert plan.lds_bytes <= 64 * 1024
    elif plan.dqk_block == 64 and plan.dv_block == 64:
        # LDS-direct kernel, narrow heads: 4 waves x 32 rows, 64-key tiles,
        # K and V rings of 2 slots each, three workgroups per CU
        assert (plan.block_m, plan.threads, plan.waves, plan.block_n) == (128, 256, 4, 64)
        assert plan.lds_bytes == (2 * 64 + 2 * 64) * 64 * 2
        assert 3 * plan.lds_bytes <= 160 * 1024
    else:
        # LDS-direct kernel, wide heads: 8 waves x 32 rows, 64-key tiles, K
        # ring of 4 slots and V ring of 2 slots (4 with the causal mask,
        # which synchronises every second tile)
        assert (plan.block_m, plan.threads, plan.waves, plan.block_n) == (256, 512, 8, 64)
        vslots = 4 if w.causal else 2
        assert plan.lds_bytes == (4 * plan.dqk_block + vslots * plan.dv_block) * 64 * 2
        assert plan.lds_bytes <= 160 * 1024
    bm = plan.block_m
    assert plan.dqk_block >= w.D_qk and plan.dv_block >= w.D_v
    assert plan.slices == w.B * w.H
    assert plan.q_blocks == math.ceil(w.S_q / bm)
    assert plan.kv_blocks == math.ceil(w.S_k / plan.block_n)
    assert plan.grid == plan.q_blocks * plan.slices
    assert plan.order == (1 if plan.slices % 8 == 0 else 0)
    total = sum(expected_tiles(qb, bm, plan.block_n, w.S_q, w.S_k, w.causal)
                for qb in range(plan.q_blocks)) * plan.slices
    assert plan.total_kv_steps == total


@pytest.mark.parametrize("B,H,S_q,D,split", [
    (1, 2, 128, 64, 4),      # 2 slices x 1 block of 128 rows
    (2, 4, 1000, 80, 4),     # 64 blocks of 128 rows
    (1, 8, 2048, 128, 4),    # 128
    (2, 16, 1920, 128, 4),   # 480: still below two per CU
    (2, 16, 2048, 128, 1),   # 512: the 128-row kernel, two workgroups per CU
    (4, 32, 4096, 64, 1),
])
def test_f32_key_split_choice(lib, B, H, S_q, D, split):
    """f32 takes the key-split kernel (32 rows per workgroup) exactly when
    the 128-row kernel would launch fewer than 512 workgroups; 16-bit inputs
    never split."""
    plan = tsd.attn_fwd_plan(B, H, S_q, 777, D, D, False, "f32")
    assert plan.key_split == split
    assert plan.block_m == (32 if split > 1 else 128)
    assert plan.grid == math.ceil(S_q / plan.block_m) * B * H
    assert tsd.attn_fwd_plan(B, H, S_q, 777, D, D, False, "bf16").key_split == 1


@pytest.mark.parametrize("B,H,S_q,S_k,causal", [
    (1, 2, 128, 128, False), (2, 4, 1000, 777, True), (2, 4, 1000, 777, False),
    (1, 8, 700, 300, True), (3, 5, 513, 1029, True), (2, 8, 1024, 1024, True),
    (1, 32, 2048, 2048, True), (1, 1, 1, 1, True),
])
def test_block_map_covers_each_tile_once(lib, B, H, S_q, S_k, causal):
    plan = tsd.attn_fwd_plan(B, H, S_q, S_k, 128, 128, causal, "bf16")
    seen = set()
    steps_in_order = []
    for blk in range(plan.grid):
        qb, sl, steps = tsd.attn_fwd_plan_block(plan, S_q, S_k, blk)
        assert 0 <= qb < plan.q_blocks and 0 <= sl < plan.slices
        assert steps == expected_tiles(qb, plan.block_m, plan.block_n, S_q, S_k, causal)
        seen.add((qb, sl))
        steps_in_order.append(steps)
        if plan.order == 1:
            # every workgroup of a slice lands on the same XCD (id % 8)
            assert sl % 8 == blk % 8
    assert len(seen) == plan.grid
    assert sum(steps_in_order) == plan.total_kv_steps
    if causal:
        # heaviest first: the work per workgroup never grows along the launch order
        assert all(a >= b for a, b in zip(steps_in_order, steps_in_order[1:]))
    with pytest.raises(tsd.TsdError):
        tsd.attn_fwd_plan_block(plan, S_q, S_k, plan.grid)


def test_vector_io_flag(lib):
    assert tsd.attn_fwd_plan(1, 1, 64, 64, 80, 80, False, "f32").vector_io == 1
    assert tsd.attn_fwd_plan(1, 1, 64, 64, 80, 80, False, "bf16").vector_io == 1
    assert tsd.attn_fwd_plan(1, 1, 64, 64, 33, 64, False, "bf16").vector_io == 0
    assert tsd.attn_fwd_plan(1, 1, 64, 64, 64, 6, False, "f32").vector_io == 0


def test_product_code_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "tiled_scaled_dot_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
                assert "liboracle" not in text and "attn_ref" not in text, f
    hdr = open(HEADER).read()
    assert "oracle" not in hdr.lower()


# ------------------------------------------------ extended entry points
# Every call below is rejected on the host before any HIP call.
MK = tsd.make_mask


def ext(q=QA, k=KA, v=VA, o=OA, lse=LA, dtype=2, mask=None, H_kv=None, **dims):
    d = dict(GOOD)
    d.update(dims)
    return tsd.attn_fwd_ext_raw(q, k, v, o, lse, d["B"], d["H"],
                                d["H"] if H_kv is None else H_kv, d["S_q"], d["S_k"],
                                d["D_qk"], d["D_v"], 0.125, 1, dtype, mask)


def part(op=OA, lp=LA, n=2, ln=64, mask=None, dtype=2, q=QA, H_kv=None, **dims):
    d = dict(GOOD)
    d.update(dims)
    return tsd.attn_fwd_partial_raw(q, KA, VA, op, lp, d["B"], d["H"],
                                    d["H"] if H_kv is None else H_kv, d["S_q"], d["S_k"],
                                    d["D_qk"], d["D_v"], 0.125, 0, dtype, mask, n, ln)


@pytest.mark.parametrize("mask,status", [
    (MK(128, kv_begin=-1), 2), (MK(128, kv_end=129), 2), (MK(128, kv_begin=50, kv_end=49), 2),
    (MK(128, window=-1), 2), (MK(128, causal_offset=(1 << 30) + 1), 3),
    (MK(128, causal_offset=-(1 << 30) - 1), 3), (MK(128, window=(1 << 30) + 1), 3),
])
def test_ext_bad_mask(lib, mask, status):
    assert ext(mask=mask) == status
    assert part(mask=mask) == status


def test_ext_fast_path_only(lib):
    assert ext(dtype=0) == 3                  # f32 inputs
    assert ext(D_qk=60, D_v=60) == 3          # widths not a multiple of 8
    assert ext(q=QA + 8) == 3                 # not 16-byte aligned
    assert ext(o=OA + 8) == 3
    assert part(dtype=0) == 3
    assert part(op=OA + 4) == 3               # f32 partial O not 16-byte aligned
    assert ext(o=None) == 1 and ext(q=None) == 1
    assert part(op=None) == 1 and part(lp=None) == 1
    assert ext(S_k=0) == 2


def test_ext_alias(lib):
    assert ext(o=KA) == 5
    assert ext(lse=OA + 64) == 5
    assert part(op=QA) == 5
    assert part(lp=VA + 16) == 5
    # the chunked output spans n times the slice outputs: chunk 1 would reach LA
    o_bytes = 1 * 2 * 128 * 64 * 4
    assert part(op=LA - o_bytes, n=2) == 5


def test_grouped_heads_rejected(lib):
    for H_kv in (0, -1, 3):                   # H = 2: 3 does not divide it
        assert ext(H_kv=H_kv) == 2
        assert part(H_kv=H_kv) == 2
    with pytest.raises(tsd.TsdError):
        tsd.attn_splitkv_plan(1, 6, 64, 1000, 64, 64, False, "bf16", None, 0, H_kv=4)
    # a group's rows form one slice: its 32-bit offsets bound H / H_kv * S_q
    assert ext(H=64, H_kv=1, S_q=1 << 18) == 3


def test_partial_bad_chunks(lib):
    assert part(n=0) == 2 and part(ln=0) == 2
    assert part(n=1 << 20, ln=1 << 12) == 3   # chunk bounds beyond int32


def merge(op=OA, lp=LA, n=3, o=VA, lse=KA, dtype=2, B=1, H=2, S_q=128, D_v=64):
    return tsd.attn_merge_raw(op, lp, n, B, H, S_q, D_v, o, lse, dtype)


def test_merge_rejects(lib):
    assert merge(op=None) == 1 and merge(lp=None) == 1 and merge(o=None) == 1
    assert merge(n=0) == 2 and merge(D_v=0) == 2 and merge(S_q=0) == 2
    assert merge(D_v=129) == 3 and merge(dtype=5) == 3
    assert merge(op=OA + 2) == 3 and merge(o=VA + 1) == 3
    assert merge(o=OA + 4096) == 5            # output inside the partial O
    assert merge(lse=LA) == 5                 # LSE on the partial LSE
    assert merge(lse=VA + 8) == 5             # LSE inside O


def test_splitkv_plan(lib):
    # few query blocks, many keys: chunks until one round of workgroups
    # covers the chip (one wide workgroup per CU)
    n, ln, ws = tsd.attn_splitkv_plan(1, 8, 512, 131072, 128, 128, False, "bf16")
    plan = tsd.attn_fwd_plan(1, 8, 512, 131072, 128, 128, False, "bf16")
    assert plan.grid * n >= 256 and plan.grid * (n - 1) < 256
    assert ln % 64 == 0 and n * ln >= 131072
    assert ws == math.ceil(n * 8 * 512 * 128 * 4 / 256) * 256 + math.ceil(n * 8 * 512 * 4 / 256) * 256
    # narrow heads: three workgroups per CU
    n, _, _ = tsd.attn_splitkv_plan(1, 8, 512, 131072, 64, 64, False, "bf16")
    plan = tsd.attn_fwd_plan(1, 8, 512, 131072, 64, 64, False, "bf16")
    assert plan.grid * n >= 768 and plan.grid * (n - 1) < 768
    # a full grid keeps one chunk and needs no workspace
    assert tsd.attn_splitkv_plan(4, 16, 4096, 4096, 128, 128, True, "bf16") == (1, 4096, 0)
    # requested counts: chunks are whole tiles and none lies past the range
    n, ln, _ = tsd.attn_splitkv_plan(1, 1, 64, 1000, 64, 64, False, "bf16", None, 7)
    assert ln == 192 and n == 6
    n, ln, _ = tsd.attn_splitkv_plan(1, 1, 64, 1000, 64, 64, False, "bf16",
                                     MK(1000, kv_begin=100, kv_end=300), 4)
    assert (n, ln) == (4, 64)
    with pytest.raises(tsd.TsdError):
        tsd.attn_splitkv_plan(1, 1, 64, 1000, 64, 64, False, "f32")
    with pytest.raises(tsd.TsdError):
        tsd.attn_splitkv_plan(1, 1, 64, 1000, 64, 64, False, "bf16", None, 300)


def test_splitkv_workspace_checks(lib):
    n, ln, ws = tsd.attn_splitkv_plan(1, 2, 128, 4096, 64, 64, False, "bf16", None, 4)
    assert n == 4 and ws > 0
    args = (QA, KA, VA, OA, LA, 1, 2, 2, 128, 4096, 64, 64, 0.125, 0, 2, None, 4)
    assert tsd.attn_fwd_splitkv_raw(*args, None, ws) == 1          # no workspace
    assert tsd.attn_fwd_splitkv_raw(*args, 0x60000000, ws - 1) == 2  # too small
    assert tsd.attn_fwd_splitkv_raw(*args, 0x60000000 + 64, ws) == 3  # not 256-aligned
    assert tsd.attn_fwd_splitkv_raw(*args, OA, ws) == 5             # workspace on O
    assert tsd.attn_fwd_splitkv_raw(*args, KA - 256, ws) == 5       # workspace into K


def test_splitkv_noalloc_host_checks(lib):
    """attn_fwd_splitkv_noalloc rejects, before any HIP call, what
    attn_fwd_splitkv rejects, and a plan whose partial results exceed the
    fixed scratch array with TSD_ERR_SCRATCH."""
    call = tsd.attn_fwd_splitkv_noalloc_raw
    good = (QA, KA, VA, OA, LA, 1, 2, 2, 128, 4096, 64, 64, 0.125, 0, 2, None, 4)
    assert call(None, *good[1:]) == 1
    assert call(*good[:3], None, *good[4:]) == 1
    assert call(*good[:14], 0, None, 4) == 3                         # f32: fast path only
    assert call(*good[:3], OA + 8, *good[4:]) == 3                   # O not 16-byte aligned
    assert call(*good[:15], MK(4096, kv_begin=-1), 4) == 2
    assert call(*good[:16], 300) == 3                                # more than 256 chunks
    # 64 heads x 4096 rows x 128 f32 columns x 64 chunks: 8 GiB of partials
    n, _, ws = tsd.attn_splitkv_plan(1, 64, 4096, 65536, 128, 128, False, "bf16", None, 64)
    assert n == 64 and ws > tsd.NOALLOC_SCRATCH_BYTES
    assert call(QA, KA, VA, OA, LA, 1, 64, 64, 4096, 65536, 128, 128, 0.125, 0, 2, None,
                64) == 7
    assert "scratch" in tsd.attn_status_string(7)


def test_planner_and_checks_from_many_threads(lib):
    """The library keeps no state: plans computed by eight host threads at
    once (ctypes drops the GIL for the call) equal the single-threaded ones,
    and invalid calls return their status from every thread."""
    import random
    from concurrent.futures import ThreadPoolExecutor
    rng = random.Random(7)
    cases = [(rng.randint(1, 4), rng.randint(1, 40), rng.randint(1, 20000), rng.randint(1, 20000),
              rng.randint(1, 128), rng.randint(1, 128), rng.random() < 0.5,
              rng.choice(["f32", "f16", "bf16"])) for _ in range(64)]
    fields = [f for f, _ in tsd.TsdPlan._fields_]

    def as_tuple(plan):
        return tuple(getattr(plan, f) for f in fields)

    want = [as_tuple(tsd.attn_fwd_plan(*c)) for c in cases]

    def worker(seed):
        r = random.Random(seed)
        for _ in range(300):
            i = r.randrange(len(cases))
            assert as_tuple(tsd.attn_fwd_plan(*cases[i])) == want[i]
            # a null Q: rejected on the host before any HIP call
            assert tsd.attn_fwd_raw(0, 16, 16, 16, 0, 1, 1, 8, 8, 64, 64, 0.1, False,
                                    "bf16") == 1   # TSD_ERR_NULL
        return True

    with ThreadPoolExecutor(8) as ex:
        assert all(ex.map(worker, range(8)))


def test_binding_rejects_tensors_on_two_devices():
    """The binding refuses a call whose tensors live on different devices
    (a kernel would otherwise read another device's memory)."""
    import torch

    a = torch.empty(1)
    b = torch.empty(1, device="meta")
    tsd._one_device(a, k=a, v=None)
    with pytest.raises(ValueError, match="meta"):
        tsd._one_device(a, k=b)


# ------------------------------------------------- planner over any sizes
from hypothesis import given, settings, strategies as st  # noqa: E402

_dims = st.one_of(st.integers(-2, 3), st.integers(1, 1 << 14), st.integers(1, 1 << 40),
                  st.sampled_from([(1 << 31) - 1, 1 << 31, (1 << 32) + 1, 1 << 62]))


@settings(max_examples=600, deadline=None)
@given(B=_dims, H=_dims, S_q=_dims, S_k=_dims, D_qk=st.integers(-1, 260),
       D_v=st.integers(-1, 260), dtype=st.integers(-1, 4), causal=st.booleans())
def test_planner_total_over_any_sizes(lib, B, H, S_q, S_k, D_qk, D_v, dtype, causal):
    """Whatever the sizes (negative, zero, up to 2^62), the planner returns a
    status instead of overflowing: SHAPE for a dimension below 1, otherwise
    OK or UNSUPPORTED, and an accepted plan fits the kernels' 32-bit grid
    and in-slice offsets."""
    try:
        plan = tsd.attn_fwd_plan(B, H, S_q, S_k, D_qk, D_v, causal, dtype)
    except tsd.TsdError as e:
        if min(B, H, S_q, S_k, D_qk, D_v) < 1:
            assert e.status == 2
        else:
            assert e.status == 3
        return
    assert min(B, H, S_q, S_k, D_qk, D_v) >= 1 and dtype in (0, 1, 2)
    elt = 4 if dtype == 0 else 2
    assert max(S_q, S_k) * max(D_qk, D_v) * elt < (1 << 31)
    assert plan.slices == B * H and plan.q_blocks == -(-S_q // plan.block_m)
    assert plan.grid == plan.q_blocks * plan.slices < (1 << 31)


@settings(max_examples=400, deadline=None)
@given(B=_dims, H_kv=st.integers(1, 64), group=st.integers(1, 64), S_q=_dims, S_k=_dims,
       D=st.sampled_from([8, 64, 128, 136]), causal=st.booleans(),
       coff=st.integers(-(1 << 31), 1 << 31), window=st.integers(-1, 1 << 31),
       n_splits=st.integers(-1, 300))
def test_splitkv_planner_total_over_any_sizes(lib, B, H_kv, group, S_q, S_k, D, causal, coff,
                                              window, n_splits):
    """The split-KV planner under the same kind of sizes and any mask values:
    a status, or a plan whose chunks cover the key range in at most 256
    whole-tile chunks."""
    H = H_kv * group
    try:
        mask = tsd.make_mask(max(S_k, 0), coff, window)
        n, ln, ws = tsd.attn_splitkv_plan(B, H, S_q, S_k, D, D, causal, "bf16", mask,
                                          n_splits, H_kv=H_kv)
    except tsd.TsdError as e:
        assert e.status in (2, 3)
        return
    assert 1 <= n <= 256 and ln % 64 == 0 and ln >= 64
    assert (n - 1) * ln < max(S_k, 1) <= n * ln or n == 1
    assert ws >= 0
