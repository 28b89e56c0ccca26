"""The oracle against its pins (CPU only), and planted mistakes against the pins.

A planted mistake is a one-line change to a private copy of the oracle's C
source (compiled into a temporary library); at least one pin must reject
each of them, which shows the pins can see that kind of error.
"""
import os
import subprocess

import pytest

import oracle
from oracle_pins import PINS

pytestmark = pytest.mark.cpu


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)


# (what the mistake is, text in attn_ref.c, replacement)
MUTATIONS = [
    ("scale dropped", "s[j] = jb->scale * dot;", "s[j] = dot;"),
    ("causal excludes the diagonal", "hi = i + jb->coff + 1;", "hi = i + jb->coff;"),
    ("wrong sign of the max shift", "l += exp(s[j] - m);", "l += exp(s[j] + m);"),
    ("V read transposed", "acc[e] += w[j] * v[j * jb->D_v + e];",
     "acc[e] += w[j] * v[e * jb->S_k + j];"),
    ("K read transposed", "dot += q[d] * k[j * jb->D_qk + d];",
     "dot += q[d] * k[d * jb->S_k + j];"),
    ("weights not normalised", "w[j] = exp(s[j] - m) / l;", "w[j] = exp(s[j] - m);"),
    ("LSE misses the max", "= m + log(l);", "= log(l);"),
    ("last feature dropped", "for (int64_t d = 0; d < jb->D_qk; ++d)",
     "for (int64_t d = 0; d + 1 < jb->D_qk; ++d)"),
    ("max seeded with 0", "double m = -INFINITY;", "double m = 0.0;"),
    ("wrong query row", "(slice * jb->S_q + i) * jb->D_qk",
     "(slice * jb->S_q + (i > 0 ? i - 1 : 0)) * jb->D_qk"),
    ("V slice stride uses D_qk", "jb->V + kv_slice * jb->S_k * jb->D_v",
     "jb->V + kv_slice * jb->S_k * jb->D_qk"),
    ("first key skipped", "for (int64_t j = lo; j < hi; ++j)\n        w[j]",
     "for (int64_t j = lo + 1; j < hi; ++j)\n        w[j]"),
    ("causal offset ignored", "hi = i + jb->coff + 1;", "hi = i + 1;"),
    ("window one key too wide", "lo = i + jb->coff - jb->window + 1;",
     "lo = i + jb->coff - jb->window;"),
    ("key range end inclusive", "int64_t lo = jb->kv_begin, hi = jb->kv_end;",
     "int64_t lo = jb->kv_begin, hi = jb->kv_end < jb->S_k ? jb->kv_end + 1 : jb->kv_end;"),
    ("key range start ignored", "int64_t lo = jb->kv_begin, hi", "int64_t lo = 0, hi"),
    ("empty row LSE zero", "jb->LSE[slice * jb->n_rows + out_row] = -INFINITY;",
     "jb->LSE[slice * jb->n_rows + out_row] = 0.0;"),
    ("K/V head by modulo", "(slice % jb->H) / (jb->H / jb->H_kv)",
     "(slice % jb->H) % jb->H_kv"),
    ("K/V batch ignored", "(slice / jb->H) * jb->H_kv +", "0 * jb->H_kv +"),
    ("query scale of the previous row's block", "i / jb->q_block]",
     "(i > 0 ? i - 1 : 0) / jb->q_block]"),
    ("key scale of the first block only", "j / jb->k_block]", "0]"),
    ("natural base instead of 2", "proto.scale = log(2.0);", "proto.scale = 1.0;"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_reject_planted_mistake(name, old, new, tmp_path):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib_path = str(tmp_path / "libmutant.so")
    oracle.build(force=True, source=str(mutant_src), output=lib_path)
    lib = oracle.load_library(lib_path)
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
        except (RuntimeError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the planted mistake: {name}"
