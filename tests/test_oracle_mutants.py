"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is a textual edit of ``oracle/vdc_oracle.c`` (a dropped term, a
wrong sign or index, a transposed operand, a wrong rounding), compiled with
gcc into a temporary directory and run against ``oracle_pins``.  The real
oracle is never modified.  Mutants only ever read inside their arrays.
"""
import os

import pytest

import oracle
import oracle_pins

# (name, text to find, replacement, which occurrence (0-based))
MUTANTS = [
    ("bias_sign", "p += b[c];", "p -= b[c];", 0),
    ("pabs_signed", "pa += fabs(term);", "pa += term;", 0),
    ("preact_tap_index", "int64_t src = t - 3 + k;", "int64_t src = t - 4 + k;", 0),
    ("preact_mask_off_by_one", "if (src < s)", "if (src <= s)", 0),
    ("dx_mask_early_stop", "if (src >= e)", "if (src >= e - 1)", 0),
    ("dx_crosses_documents", "if (src >= e)", "if (src >= S)", 0),
    ("dx_weight_transposed", "v += w[c * 4 + k] * dpre[src * C + c];",
     "v += w[c * 4 + 3 - k] * dpre[src * C + c];", 0),
    ("dx_drops_tap", "for (int k = 0; k < 4; k++) {\n                        int64_t src = t + 3 - k;",
     "for (int k = 1; k < 4; k++) {\n                        int64_t src = t + 3 - k;", 0),
    ("silu_grad_sign", "return s * (1.0 + z * (1.0 - s));", "return s * (1.0 - z * (1.0 - s));", 0),
    ("silu_grad_drops_term", "return s * (1.0 + z * (1.0 - s));", "return s * (1.0 + z);", 0),
    ("silu_drops_z", "return z * sigmoid(z);", "return sigmoid(z);", 0),
    ("sigmoid_sign", "return 1.0 / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(z));", 0),
    ("policy_ignored", "double z = policy == ORC_POLICY_BF16 ? bf16_round_value(p) : p;",
     "double z = p;", 0),
    ("policy_swapped", "double z = policy == ORC_POLICY_BF16 ? bf16_round_value(p) : p;",
     "double z = policy == ORC_POLICY_FP32 ? bf16_round_value(p) : p;", 0),
    ("dw_tap_index", "int64_t src = t - 3 + k;", "int64_t src = t - 4 + k;", 1),
    ("dw_mask_off_by_one", "if (src < s)", "if (src <= s)", 1),
    ("dw_uses_dy", "double g = dpre[t * C + c];", "double g = dy[t * C + c];", 0),
    ("dw_transposed_store", "dw_out[c * 4 + k] = nsum_value(&acc[c * 5 + k]);",
     "dw_out[c * 4 + k] = nsum_value(&acc[c * 5 + 3 - k]);", 0),
    ("db_weighted_by_x", "nsum_add(&acc[c * 5 + 4], g);", "nsum_add(&acc[c * 5 + 4], g * x[t * C + c]);", 0),
    ("bf16_extra_bit", "int qexp = e - 8;", "int qexp = e - 9;", 0),
    ("bf16_ties_away", "ldexp(nearbyint(ldexp(a, -qexp))", "ldexp(round(ldexp(a, -qexp))", 0),
    ("bf16_subnormal_quantum", "qexp = -133;", "qexp = -132;", 0),
    ("bf16_decode_shift", "(uint32_t)in[i] << 16", "(uint32_t)in[i] << 15", 0),
]


def _mutate(src, find, repl, occurrence):
    pos = -1
    for _ in range(occurrence + 1):
        pos = src.find(find, pos + 1)
        assert pos >= 0, "mutation anchor not found: %r (occurrence %d)" % (find, occurrence)
    return src[:pos] + repl + src[pos + len(find):]


@pytest.mark.parametrize("name,find,repl,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, find, repl, occ, tmp_path):
    src = open(oracle.SOURCE).read()
    mutated = _mutate(src, find, repl, occ)
    assert mutated != src
    c_path = os.path.join(tmp_path, "mutant_%s.c" % name)
    so_path = os.path.join(tmp_path, "libmutant_%s.so" % name)
    with open(c_path, "w") as fh:
        fh.write(mutated)
    oracle.compile_library(c_path, so_path)
    caught = oracle_pins.first_failure(oracle.Oracle(so_path))
    assert caught is not None, "mutant %s passed every pin" % name
