"""The pins are strong enough: plausible mistakes planted in a copy of the C
oracle (on the CPU, in a temporary build) must each fail at least one pin.

Nothing here touches the real oracle library or the GPU path; each mutant is a
text edit of ``oracle/hd_oracle.c`` compiled into a temporary directory.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "hd_oracle.c")
INTRA, CROSS = 0, 1

MUTANTS = [
    ("intra sees one future token", "if (ik > iq) return 0;", "if (ik > iq + 1) return 0;",
     [pins.test_golden_masks_figure2, pins.test_mask_exhaustive_c_vs_onebased]),
    ("intra drops the diagonal", "if (ik > iq) return 0;", "if (ik >= iq && iq > 0) return 0;",
     [pins.test_golden_masks_figure2]),
    ("streams not separated", "if (sk != sq) return 0;", "",
     [pins.test_intra_is_n_independent_causal]),
    ("intra window off by one", "if (W > 0 && iq - ik >= W) return 0;",
     "if (W > 0 && iq - ik > W) return 0;", [pins.test_golden_masks_figure2]),
    ("cross window in tokens, not positions", "tq - tk >= (int64_t)n * W", "tq - tk >= W",
     [pins.test_golden_masks_figure2, lambda o: pins.test_windows_are_banded_sdpa(o, 2)]),
    ("GQA head map modulo", "int64_t hk = h / g;", "int64_t hk = h % Hkv;",
     [pins.test_gqa_equals_repeated_mha]),
    ("scale dropped", "scores[j] = scale * dot;", "scores[j] = dot;",
     [lambda o: pins.test_n1_is_textbook_causal(o, CROSS)]),
    ("key head offset dropped", "koff[tk] = ((b * nL + tk) * Hkv + hk) * d;",
     "koff[tk] = ((b * nL + tk) * Hkv) * d;",
     [lambda o: pins.test_n1_is_textbook_causal(o, INTRA), pins.test_c_oracle_matches_brute_force]),
    ("value read from key", "o[c] += p * load_elem(v, dtype, krow_off[j] + c);",
     "o[c] += p * load_elem(k, dtype, krow_off[j] + c);",
     [pins.test_worked_example_closed_form]),
    ("lse without max shift", "*lse = m + log(l);", "*lse = log(l);",
     [pins.test_lse_matches_logsumexp_and_scale]),
    ("decode reads stale cache row for the new token", "if (tok < len) {", "if (tok <= len && tok < T_cap) {",
     [lambda o: pins.test_decode_equals_prefill_rows(o, CROSS, 0)]),
    ("expansion stream-major", "(((int64_t)b * L + i) * n + s) * row_bytes",
     "(((int64_t)b * n + s) * L + i) * row_bytes", [pins.test_expand_golden_order]),
    ("bwd dQ accumulates value rows", "out[c] += scale * ds * load_elem(k, dtype, koff + c);",
     "out[c] += scale * ds * load_elem(v, dtype, koff + c);",
     [lambda o: pins.test_bwd_matches_autograd(o, CROSS, 0, 1),
      lambda o: pins.test_bwd_finite_differences(o, INTRA, 0)]),
    ("bwd dK drops the scale", "gk[c] += scale * ds * load_elem(q, dtype, qoff + c);",
     "gk[c] += ds * load_elem(q, dtype, qoff + c);",
     [lambda o: pins.test_bwd_matches_autograd(o, INTRA, 2, 2)]),
    ("bwd dV weighted by dS", "gv[c] += p * load_elem(dout, dtype, qoff + c);",
     "gv[c] += ds * load_elem(dout, dtype, qoff + c);",
     [lambda o: pins.test_bwd_invariants(o, CROSS, 0), pins.test_bwd_zero_query_closed_form]),
    ("bwd key rows skip their own query", "for (int64_t t = tk; t < nL; ++t) {",
     "for (int64_t t = tk + 1; t < nL; ++t) {", [pins.test_bwd_window1_closed_form]),
    ("rope rotates the wrong way", "out[row + c] = x0 * co - x1 * si;", "out[row + c] = x0 * co + x1 * si;",
     [pins.test_rope_matches_transformers_rotate_half, pins.test_rope_golden_d4]),
    ("rope frequency exponent off by one", "const double f = pow(theta, -2.0 * c / d);",
     "const double f = pow(theta, -2.0 * (c + 1) / d);",
     [pins.test_rope_matches_transformers_rotate_half, pins.test_rope_golden_d4]),
    ("rope decode position ignores the stream", "const double pos = (double)(t * t_mul + t_add) +",
     "const double pos = (double)(0 * t * t_mul + t_add) +", [pins.test_rope_decode_positions]),
    ("rope row offset dropped", "const double pos = (double)(t * t_mul + t_add) +",
     "const double pos = (double)(t * t_mul) +", [pins.test_rope_final_stream_and_final_decode_positions]),
    ("final query placed at stream 0", "int64_t t = i * n + (n - 1);   /* the final stream's expanded position */",
     "int64_t t = i * n;   /* the final stream's expanded position */",
     [lambda o: pins.test_final_matches_sdpa_with_onebased_rows(o, CROSS, 0), pins.test_final_closed_forms]),
    ("final keys stop before the token's other streams",
     "int64_t nk = t + 1;            /* every mask is causal: t_k <= t */",
     "int64_t nk = i * n + 1;            /* every mask is causal: t_k <= t */",
     [lambda o: pins.test_final_matches_sdpa_with_onebased_rows(o, CROSS, 0),
      lambda o: pins.test_final_equals_full_layer_last_stream_rows(o, CROSS, 2)]),
    ("final lse stored query-major", "lse[(b * Hq + h) * L + i] = lrow[r];", "lse[(b * L + i) * Hq + h] = lrow[r];",
     [lambda o: pins.test_final_matches_sdpa_with_onebased_rows(o, INTRA, 2)]),
    ("final bwd dq stops before the token's other streams", "for (int64_t tk = 0; tk <= tq; ++tk) {",
     "for (int64_t tk = 0; tk <= i * n; ++tk) {",
     [lambda o: pins.test_final_bwd_matches_autograd(o, CROSS, 0, 2)]),
    ("final bwd keys skip the query of their own token", "if (tq < tk || !oracle_visible(tq, tk, n, mode, W)) continue;",
     "if (tq <= tk || !oracle_visible(tq, tk, n, mode, W)) continue;",
     [lambda o: pins.test_final_bwd_matches_autograd(o, INTRA, 0, 1), lambda o: pins.test_final_bwd_invariants(o, INTRA, 0)]),
    ("final bwd D read from the lse slot", "double lse_i = lse[(b * Hq + h) * L + i], D_i = Drow[(b * Hq + h) * L + i];\n        double *gq",
     "double lse_i = lse[(b * Hq + h) * L + i], D_i = lse[(b * Hq + h) * L + i];\n        double *gq",
     [lambda o: pins.test_final_bwd_matches_autograd(o, CROSS, 2, 3)]),
]


@pytest.mark.parametrize("name,old,new,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, checks):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for '{name}' must occur once"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    lib_path = str(tmp_path / "libmut.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(mut), "-o", lib_path, "-lm"],
                   check=True)
    lib = oracle._configure(ctypes.CDLL(lib_path))
    saved = oracle._load()
    oracle._lib = lib
    try:
        for check in checks:
            with pytest.raises((AssertionError, ValueError)):
                check(oracle)
    finally:
        oracle._lib = saved
