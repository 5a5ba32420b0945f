"""Planted mistakes in the oracle must fail its pins.

Each case copies oracle/msa_oracle.c, applies one plausible mistake (a
dropped term, an off-by-one, a wrong index or operand), compiles the copy
with gcc into a temporary library, points the oracle binding at it and runs
the pins of test_oracle_pins.py: at least one must fail.  Nothing here
touches a GPU.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle_backward as bwd_pins
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "msa_oracle.c")

MUTANTS = {
    # scores see key t+0 only up to t-1 (breaks causality inside the own block)
    "causal_strict": ("j < start + (b + 1) * ORC_BS && j <= t; ++j) {\n                    double dot",
                      "j < start + (b + 1) * ORC_BS && j < t; ++j) {\n                    double dot"),
    # block score summed instead of max-reduced
    "sum_not_max": ("if (dot > best) best = dot;\n                }\n                row[b] = best;\n            }\n        }\n    }\n    return bad",
                    "best = (best == -INFINITY ? 0.0 : best) + dot;\n                }\n                row[b] = best;\n            }\n        }\n    }\n    return bad"),
    # local window one block too wide
    "local_off_by_one": ("(b >= c - local + 1)", "(b >= c - local)"),
    # init range one block too wide
    "init_off_by_one": ("(b < init)", "(b <= init)"),
    # ties prefer the higher block id
    "ties_reversed": ("(x->b > y->b) - (x->b < y->b)", "(x->b < y->b) - (x->b > y->b)"),
    # query head -> KV head by h % 4 instead of contiguous groups
    "gqa_interleaved": ("int h = g * ORC_GROUP + hh;\n                    attend_keys(q + ((size_t)t",
                        "int h = hh * ORC_KVH + g;\n                    attend_keys(q + ((size_t)t"),
    # key blocks aligned to the packed batch instead of the document
    "global_block_ids": ("int blk = (j - start) / ORC_BS, sel = 0;", "int blk = j / ORC_BS, sel = 0;"),
    # softmax scale dropped
    "no_scale": ("z[j] = scale * dot;", "z[j] = dot;"),
    # decode ignores the page table
    "no_page_table": ("return (size_t)pt[(size_t)r * max_pages + j / ORC_BS] * ORC_BS + (size_t)(j % ORC_BS);",
                      "return (size_t)j + 0 * (size_t)pt[0] * (size_t)max_pages * (size_t)r;"),
    # E4M3 exponent bias off by one
    "e4m3_bias": ("ldexp(8.0 + m, e - 10)", "ldexp(8.0 + m, e - 11)"),
    # backward: softmax scale dropped from dq
    "bwd_dq_no_scale": ("dqr[x] += scale * ds * bf16_value(kr[x]);", "dqr[x] += ds * bf16_value(kr[x]);"),
    # backward: the D term dropped from dS (rows, then keys)
    "bwd_rows_no_D": ("double ds = exp(z[a] - l) * (dp[a] - Dth);", "double ds = exp(z[a] - l) * dp[a];"),
    "bwd_keys_no_D": ("double ds = p * (dot_bf16(dor, vr) - D[(size_t)t * ORC_QH + h]);",
                      "double ds = p * dot_bf16(dor, vr);"),
    # backward: dv weighted by dS instead of P
    "bwd_dv_uses_ds": ("dvr[x] += p * bf16_value(dor[x]);", "dvr[x] += ds * bf16_value(dor[x]);"),
    # backward: dk built from the key instead of the query (wrong operand)
    "bwd_dk_wrong_operand": ("dkr[x] += scale * ds * bf16_value(qr[x]);",
                             "dkr[x] += scale * ds * bf16_value(kr[x]);"),
    # backward: log-sum-exp without its max shift
    "bwd_lse_no_max": ("double l = zmax + log(sum);", "double l = log(sum);"),
    # backward: key t excluded from its own row
    "bwd_strict_causal": ("if (j > t || j < start) return 0;", "if (j >= t || j < start) return 0;"),
    # backward: query head -> KV head interleaved in the per-key phase
    "bwd_keys_gqa_interleaved": (
        "int h = g * ORC_GROUP + hh;\n                    const uint16_t *qr = q + ((size_t)t * ORC_QH + h) * ORC_D;\n"
        "                    const uint16_t *dor = dout + ((size_t)t * ORC_QH + h) * ORC_D;\n                    double p",
        "int h = hh * ORC_KVH + g;\n                    const uint16_t *qr = q + ((size_t)t * ORC_QH + h) * ORC_D;\n"
        "                    const uint16_t *dor = dout + ((size_t)t * ORC_QH + h) * ORC_D;\n                    double p"),
}

# pins of the backward oracle (tests/test_oracle_backward.py), run without arguments
BACKWARD_PINS = ["test_dense_reduction_matches_autograd", "test_sparse_rows_match_autograd_and_forward",
                 "test_invariants_and_single_key_row"]

PIN_TESTS = [
    ("test_e4m3_decoder_matches_torch_on_all_codes", {}),
    ("test_scores_equal_dense_brute_force", {"index_dtype": "bf16"}),
    ("test_scores_equal_dense_brute_force", {"index_dtype": "fp8"}),
    ("test_scores_closed_form_increasing", {}),
    ("test_selection_brute_force_subsets", {}),
    ("test_selection_invariants_and_margin", {}),
    ("test_dense_reduction_equals_sdpa", {}),
    ("test_sparse_attention_equals_masked_sdpa", {}),
    ("test_attention_closed_forms", {}),
    ("test_decode_page_permutation_invariance", {}),
    ("test_decode_dense_reduction_equals_sdpa", {}),
]


def _golden_all(orc):
    for case in pins._golden_cases():
        pins.test_selection_golden(orc, case)


def _build_mutant(tmp_path, name, old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-shared", "-fPIC",
                    "-std=c11", "-o", str(so), str(src), "-lm"], check=True)
    return str(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    so = _build_mutant(tmp_path, name, old, new)
    oracle.lib()                                  # make sure the real one is configured
    real = oracle._lib
    mutant = ctypes.CDLL(so)
    # copy argtypes/restypes of every exported oracle function
    for sym in ("oracle_bf16_value", "oracle_e4m3_value", "oracle_query_blocks", "oracle_scores",
                "oracle_select", "oracle_attend", "oracle_decode_query_blocks",
                "oracle_decode_scores", "oracle_decode_attend", "oracle_num_threads",
                "oracle_attend_backward_rows", "oracle_attend_backward_keys"):
        f_real, f_mut = getattr(real, sym), getattr(mutant, sym)
        f_mut.argtypes = f_real.argtypes
        f_mut.restype = f_real.restype
    monkeypatch.setattr(oracle, "_lib", mutant)
    checks = [(n, (lambda n=n, kw=kw: getattr(pins, n)(oracle, **kw))) for n, kw in PIN_TESTS]
    checks.insert(1, ("test_selection_golden", lambda: _golden_all(oracle)))
    checks += [(n, getattr(bwd_pins, n)) for n in BACKWARD_PINS]
    caught_by = None
    for test_name, run in checks:
        try:
            run()
        except AssertionError:
            caught_by = test_name
            break
    assert caught_by is not None, f"mutant {name} passed every pin"
