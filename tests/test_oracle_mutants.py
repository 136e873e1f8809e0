"""Each plausible mistake planted in a copy of the oracle (on the CPU) must
fail at least one pin. This shows the pins constrain every part of the oracle:
mask rules, block classification, scale, soft-cap order, normalisation, the
logsumexp base, operand indexing and the empty-row convention."""
import os

import pytest

import oracle
import oracle_pins

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("causal_direction", "      return i >= j;\n", "      return i <= j;\n"),
    ("window_inclusive", "(i - j) < window", "(i - j) <= window"),
    ("document_without_causal", "return i >= j && doc[i] == doc[j];", "return doc[i] == doc[j];"),
    ("dropped_scale", "double sc = dot * scale;", "double sc = dot;"),
    ("softcap_before_scale",
     "double sc = dot * scale;\n    if (softcap > 0.0) sc = softcap * tanh(sc / softcap);",
     "double sc = dot;\n    if (softcap > 0.0) sc = softcap * tanh(sc / softcap);\n"
     "    sc *= scale;"),
    ("lse_log2", "lse[n] = m + log(l);", "lse[n] = m + log2(l);"),
    ("missing_normalisation", "for (int64_t e = 0; e < Ev; ++e) o[e] /= l;", ""),
    ("transposed_k", "dot += qi[e] * kh[j * E + e]", "dot += qi[e] * kh[e * S + j]"),
    ("reversed_v", "vh[j * Ev + e]", "vh[(S - 1 - j) * Ev + e]"),
    ("full_threshold", "if (count == bs * bs)", "if (count * 2 >= bs * bs)"),
    ("pad_minus_one", "      kv_idx[qb * nk + t] = 0;", "      kv_idx[qb * nk + t] = -1;"),
    ("block_row_off_by_one", "i < (qb + 1) * bs && i < L", "i <= (qb + 1) * bs && i < L"),
    ("empty_row_lse_zero", "        lse[n] = -INFINITY;\n        continue;",
     "        lse[n] = 0.0;\n        continue;"),
    ("max_not_subtracted_in_lse", "lse[n] = m + log(l);", "lse[n] = log(l);"),
    ("lower_right_offset_sign", "return i + (S - L) >= j;", "return i + (L - S) >= j;"),
    ("sliding_lower_right_unshifted", "const int64_t p = i + (S - L);", "const int64_t p = i;"),
    ("padding_end_ignored", "|| j < kept_lo || j >= kept_hi)", "|| j < kept_lo)"),
    ("padding_end_inclusive", "|| j < kept_lo || j >= kept_hi)", "|| j < kept_lo || j > kept_hi)"),
    ("padding_start_ignored", "|| j < kept_lo || j >= kept_hi)", "|| j >= kept_hi)"),
    ("dense_transposed", "return dense[i * S + j] != 0;", "return dense[j * L + i] != 0;"),
    ("dense_inverted", "return dense[i * S + j] != 0;", "return dense[i * S + j] == 0;"),
    ("pack_bit_order", "word |= (uint32_t)1 << b;", "word |= (uint32_t)1 << (31 - b);"),
    ("pack_words_per_row", "const int64_t W = 4 * ((S + 127) / 128);", "const int64_t W = (S + 31) / 32;"),
    ("bwd_drops_row_term", "double ds = p * (dp - D) * scale;", "double ds = p * dp * scale;"),
    ("bwd_drops_scale", "double ds = p * (dp - D) * scale;", "double ds = p * (dp - D);"),
    ("bwd_drops_softcap_derivative",
     "if (softcap > 0.0) ds *= 1.0 - (sp / softcap) * (sp / softcap);", ""),
    ("bwd_dv_from_ds", "dvh[j * E + e] += p[j] * doi[e];", "dvh[j * E + e] += ds * doi[e];"),
    ("bwd_dk_from_dout", "dkh[j * E + e] += ds * qi[e];", "dkh[j * E + e] += ds * doi[e];"),
    ("bidirectional_keeps_causal", "      return doc[i] == doc[j];\n",
     "      return i >= j && doc[i] == doc[j];\n"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, old, new):
    assert source.count(old) == 1, f"mutation anchor for {name} not unique in oracle.c"
    src = tmp_path / f"{name}.c"
    src.write_text(source.replace(old, new))
    lib = oracle.compile_source(str(src), str(tmp_path / f"lib{name}.so"))
    orc = oracle.Oracle(lib)
    failures = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, ValueError, RuntimeError, FloatingPointError) as e:
            failures.append(check.__name__)
            break
    assert failures, f"mutant {name} passed every pin"
    os.remove(lib)
