"""Planted mistakes in the oracle must fail at least one pin (CPU only).

Each mutation below is a plausible slip — a dropped term, a wrong sign or
index, a transposed operand, a wrong split formula. The test patches a copy of
oracle/oracle.c, builds it into a temporary library, runs every pin of
tests/oracle_pins.py on it, and requires at least one pin to fail. This shows
the pins would catch such a mistake in the real oracle.
"""
import os
import tempfile

import pytest

import oracle
import oracle_pins
from oracle import build as oracle_build

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement)
MUTATIONS = [
    ("scale_dropped", "s[j] = scale * acc;", "s[j] = acc;"),
    ("diagonal_excluded", "if (kp > qp) return 0; ", "if (kp >= qp) return 0; "),
    ("mask_reversed", "if (kp > qp) return 0; ", "if (kp < qp) return 0; "),
    ("document_start_ignored", "if (q_start && kp < q_start[i]) return 0;", ";"),
    ("gqa_modulo_mapping", "int32_t g = h / group;", "int32_t g = h % hkv;"),
    ("k_layout_transposed", "load_value(k, in_dtype, (j * hkv + g) * (int64_t)d + t)",
     "load_value(k, in_dtype, (g * lk + j) * (int64_t)d + t)"),
    ("q_reads_kv_head", "(i * hq + h) * (int64_t)d + t", "(i * hq + h / (hq / hkv)) * (int64_t)d + t"),
    ("v_head_fixed", "int32_t g = h / (hq / hkv);\n            for (int64_t j = 0; j < lk; ++j) {",
     "int32_t g = 0;\n            for (int64_t j = 0; j < lk; ++j) {"),
    ("lse_without_max", "lse[n] = m + log(l);", "lse[n] = log(l);"),
    ("output_not_normalised", "for (int32_t t = 0; t < d; ++t) on[t] /= l;", ";"),
    ("exponent_sign", "if (s[j] != -INFINITY) l += exp(s[j] - m);", "if (s[j] != -INFINITY) l += exp(m - s[j]);"),
    ("zigzag_second_chunk", "second = 2 * cp - 1 - rank;", "second = 2 * cp - 2 - rank;"),
    ("zigzag_chunk_order", "int64_t first = rank, second", "int64_t first = 2 * cp - 1 - rank, second"),
    ("striped_offset", "for (int64_t t = rank; t < len; t += cp)", "for (int64_t t = cp - 1 - rank; t < len; t += cp)"),
    ("contiguous_stride", "out_pos[n++] = (int32_t)(base + rank * per + t);",
     "out_pos[n++] = (int32_t)(base + rank + t * cp);"),
    ("doc_base_not_advanced", "base += doc_lens[t];", ";"),
    ("merge_weights_swapped", "wa = exp(la - L);\n            wb = exp(lb - L);",
     "wa = exp(lb - L);\n            wb = exp(la - L);"),
    ("merge_lse_max_only", "L = mx + log(exp(la - mx) + exp(lb - mx));", "L = mx;"),
    ("merge_empty_unguarded", "if (la == -INFINITY && lb == -INFINITY) {", "if (0) {"),
    ("bf16_widening_shift", "<< 16;", "<< 15;"),
    ("grad_delta_dropped", "double ds = p * (dp - di);", "double ds = p * dp;"),
    ("grad_delta_from_dout", "di += dorow[t] * orow[t];", "di += dorow[t] * dorow[t];"),
    ("grad_dq_sign", "dq[n * d + t] += scale * ds *", "dq[n * d + t] -= scale * ds *"),
    ("grad_dq_reads_v", "dq[n * d + t] += scale * ds * load_value(k, in_dtype, kv + t);",
     "dq[n * d + t] += scale * ds * load_value(v, in_dtype, kv + t);"),
    ("grad_dk_unscaled", "if (dkj) dkj[t] += scale * ds *", "if (dkj) dkj[t] += ds *"),
    ("grad_dv_weighted_by_ds", "if (dvj) dvj[t] += p * dorow[t];", "if (dvj) dvj[t] += ds * dorow[t];"),
    ("grad_key_pass_lse_sign", "double p = exp(scale * acc - lse[n]);", "double p = exp(scale * acc + lse[n]);"),
    ("grad_key_pass_one_head", "for (int32_t h = g * group; h < (g + 1) * group; ++h)",
     "for (int32_t h = g; h < g + 1; ++h)"),
    ("grad_key_pass_unmasked",
     "if (!key_visible(causal, q_pos ? q_pos[i] : 0, q_start, i, k_pos ? k_pos[j] : 0)) continue;", ";"),
    ("grad_normaliser_sign", "if (s[j] != -INFINITY) z += exp(s[j] - m);",
     "if (s[j] != -INFINITY) z += exp(m - s[j]);"),
    ("grad_row_lse_without_max", "lse[n] = m + log(z);", "lse[n] = log(z);"),
    ("grad_key_pass_stale_delta", "double ds = p * (dp - dd[n]);", "double ds = p * (dp - dd[0]);"),
]


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(workdir, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation %s no longer matches oracle.c exactly once" % name
    path = os.path.join(workdir, name + ".c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle_build.build(src=path, out=os.path.join(workdir, "lib%s.so" % name),
                             extra_flags=("-w", "-I", os.path.dirname(SRC)))
    orc = oracle.Oracle(lib)
    failed = None
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed = pin.__name__
            break
    assert failed, "planted mistake %s passed every pin" % name
