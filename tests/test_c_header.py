"""The C ABI from C: `include/tsd_attn.h` compiles as strict C99 and as
C++17 with every warning an error, a program built against it links
libtsd_attn.so, and its host-only calls (the planners, the status text and
the argument checks that return before any HIP call) give what the Python
binding reports for the same arguments.  No GPU is needed."""
import os
import shutil
import subprocess

import pytest

import tiled_scaled_dot_amd as tsd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

PROGRAM = r"""
#include "tsd_attn.h"

#include <stdint.h>
#include <stdio.h>

int main(void)
{
    tsd_plan p;
    tsd_mask m;
    int64_t n = 0, len = 0, ws = 0, qb = 0, sl = 0, steps = 0;
    int st = attn_fwd_plan(1, 32, 16384, 16384, 128, 128, 1, TSD_BF16, &p);
    if (st != TSD_OK) return 10 + st;
    printf("plan %d %d %d %lld %lld %lld\n", p.block_m, p.block_n, p.threads,
           (long long)p.q_blocks, (long long)p.grid, (long long)p.total_kv_steps);
    st = attn_fwd_plan_block(&p, 16384, 16384, 5, &qb, &sl, &steps);
    if (st != TSD_OK) return 20 + st;
    printf("block %lld %lld %lld\n", (long long)qb, (long long)sl, (long long)steps);
    m.causal_offset = 16383;
    m.window = 0;
    m.kv_begin = 0;
    m.kv_end = 16384;
    st = attn_splitkv_plan(4, 32, 8, 1, 16384, 128, 128, 1, TSD_BF16, &m, 0, &n, &len, &ws);
    if (st != TSD_OK) return 30 + st;
    printf("splitkv %lld %lld %lld\n", (long long)n, (long long)len, (long long)ws);
    /* argument checks that return before any HIP call */
    printf("null %d\n", attn_fwd(NULL, NULL, NULL, NULL, NULL, 1, 1, 1, 1, 1, 1, 1.0f, 0,
                                 TSD_BF16, NULL));
    printf("shape %d\n", attn_fwd_plan(0, 1, 1, 1, 1, 1, 0, TSD_BF16, &p));
    printf("width %d\n", attn_fwd_plan(1, 1, 1, 1, 129, 64, 0, TSD_BF16, &p));
    printf("scratch %lld\n", (long long)TSD_NOALLOC_SCRATCH_BYTES);
    printf("text %s\n", attn_status_string(TSD_ERR_UNSUPPORTED));
    return 0;
}
"""


def compiler(name):
    path = shutil.which(name)
    if path is None:
        pytest.skip(f"{name} not found")
    return path


@pytest.fixture(scope="module")
def lib_path():
    tsd.library()   # raises if the library is not built
    return tsd.LIBRARY_PATH


@pytest.mark.parametrize("cc,std,suffix", [("gcc", "-std=c99", "c"), ("g++", "-std=c++17", "cpp")])
def test_header_compiles_links_and_plans(tmp_path, lib_path, cc, std, suffix):
    src = tmp_path / f"use_abi.{suffix}"
    src.write_text(PROGRAM)
    exe = tmp_path / f"use_abi_{suffix}"
    libdir = os.path.dirname(lib_path)
    cmd = [compiler(cc), std, "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INCLUDE,
           str(src), "-o", str(exe), lib_path, f"-Wl,-rpath,{libdir}"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stdout, run.stderr)
    got = dict(line.split(" ", 1) for line in run.stdout.strip().splitlines())

    plan = tsd.attn_fwd_plan(1, 32, 16384, 16384, 128, 128, True, "bf16")
    assert got["plan"].split() == [str(x) for x in (plan.block_m, plan.block_n, plan.threads,
                                                    plan.q_blocks, plan.grid,
                                                    plan.total_kv_steps)]
    assert got["block"].split() == [str(x) for x in
                                     tsd.attn_fwd_plan_block(plan, 16384, 16384, 5)]
    n, ln, ws = tsd.attn_splitkv_plan(4, 32, 1, 16384, 128, 128, True, "bf16",
                                      tsd.make_mask(16384, 16383), 0, H_kv=8)
    assert got["splitkv"].split() == [str(n), str(ln), str(ws)]
    code = {name: num for num, name in tsd.STATUS.items()}
    assert int(got["null"]) == code["TSD_ERR_NULL"]
    assert int(got["shape"]) == code["TSD_ERR_SHAPE"]
    assert int(got["width"]) == code["TSD_ERR_UNSUPPORTED"]
    assert int(got["scratch"]) == tsd.NOALLOC_SCRATCH_BYTES
    assert got["text"] == tsd.attn_status_string(code["TSD_ERR_UNSUPPORTED"])
