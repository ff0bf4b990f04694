"""Plants plausible mistakes in copies of the oracle and checks that the pins catch each one.

Every mutant is the oracle source with one textual change (a dropped term, a
wrong sign, a wrong or transposed index, an ignored argument), compiled with
g++ into a temporary library. The pins of oracle_checks.py must fail on every
mutant; a mutant that survives means a mistake of that kind would go unnoticed.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle
from oracle_checks import CHECKS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.cpp")

# (name, original text, replacement, which occurrence of the original text)
MUTATIONS = [
    ("dense_drops_v", "const double vi = (v == nullptr) ? 1.0 : val((double)v[i], absolute);",
     "const double vi = 1.0;", 0),
    ("csr_drops_v", "const double vi = (v == nullptr) ? 1.0 : val((double)v[i], absolute);",
     "const double vi = 1.0;", 1),
    ("beta_term_sign", "if (beta != 0.0f) r += val((double)beta, absolute)",
     "if (beta != 0.0f) r -= val((double)beta, absolute)", 0),
    ("beta_not_applied", "r += val((double)beta, absolute) * val((double)z[j], absolute);",
     "r += val((double)z[j], absolute);", 0),
    ("alpha_dropped", "double r = val((double)alpha, absolute) * S[j];", "double r = S[j];", 0),
    ("dense_dot_drops_last_term", "for (int64_t k = 0; k < n; ++k) t +=",
     "for (int64_t k = 0; k + 1 < n; ++k) t +=", 0),
    ("dense_dot_wrong_y_index", "val(elem(row[k]), absolute) * val((double)y[k], absolute)",
     "val(elem(row[k]), absolute) * val((double)y[n - 1 - k], absolute)", 0),
    ("dense_transpose_wrong_column", "S[(size_t)j] += val(elem(row[j]), absolute) * ui;",
     "S[(size_t)j] += val(elem(row[n - 1 - j]), absolute) * ui;", 0),
    ("dense_step1_ignores_ldx", "const Elem* row = X + i * ldx;", "const Elem* row = X + i * n;", 0),
    ("dense_step3_ignores_ldx", "const Elem* row = X + i * ldx;", "const Elem* row = X + i * n;", 1),
    ("bf16_widened_by_15_bits", "const uint32_t b = (uint32_t)h << 16;", "const uint32_t b = (uint32_t)h << 15;", 0),
    ("bf16_read_as_low_half", "const uint32_t b = (uint32_t)h << 16;", "const uint32_t b = (uint32_t)h;", 0),
    ("bf16_sign_dropped", "const uint32_t b = (uint32_t)h << 16;", "const uint32_t b = (uint32_t)(h & 0x7fff) << 16;",
     0),
    ("csr_gathers_y_by_row", "val((double)y[col_idx[p]], absolute)", "val((double)y[i % n], absolute)", 0),
    ("csr_scatters_by_row", "S[(size_t)col_idx[p]] +=", "S[(size_t)(i % n)] +=", 0),
    ("csr_drops_repeated_column",
     "t += val((double)values[p], absolute) * val((double)y[col_idx[p]], absolute);",
     "if (p == row_ptr[i] || col_idx[p] != col_idx[p - 1]) "
     "t += val((double)values[p], absolute) * val((double)y[col_idx[p]], absolute);", 0),
    ("csr_skips_first_entry", "for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p)",
     "for (int64_t p = row_ptr[i] + 1; p < row_ptr[i + 1]; ++p)", 0),
    ("quick_return_ignores_beta", "(beta == 0.0f) ? 0.0 : val((double)beta, absolute) * val((double)z[j], absolute)",
     "(beta == 0.0f) ? 0.0 : val((double)z[j], absolute)", 0),
    ("bound_keeps_signs", "return absolute ? std::fabs(x) : x;", "return x;", 0),
    # the CSR normaliser alone (every CSR parity verdict divides by it)
    ("csr_bound_y_keeps_sign", "t += val((double)values[p], absolute) * val((double)y[col_idx[p]], absolute);",
     "t += val((double)values[p], absolute) * (double)y[col_idx[p]];", 0),
    ("csr_bound_step1_values_keep_sign",
     "t += val((double)values[p], absolute) * val((double)y[col_idx[p]], absolute);",
     "t += (double)values[p] * val((double)y[col_idx[p]], absolute);", 0),
    ("csr_bound_step3_values_keep_sign", "S[(size_t)col_idx[p]] += val((double)values[p], absolute) * ui;",
     "S[(size_t)col_idx[p]] += (double)values[p] * ui;", 0),
    ("csr_bound_v_keeps_sign", "const double vi = (v == nullptr) ? 1.0 : val((double)v[i], absolute);",
     "const double vi = (v == nullptr) ? 1.0 : (double)v[i];", 1),
    ("bound_beta_keeps_sign", "r += val((double)beta, absolute) * val((double)z[j], absolute);",
     "r += (double)beta * val((double)z[j], absolute);", 0),
    ("bound_z_keeps_sign", "r += val((double)beta, absolute) * val((double)z[j], absolute);",
     "r += val((double)beta, absolute) * (double)z[j];", 0),
    # the two halves
    ("rowdot_drops_v", "const double vi = (v == nullptr) ? 1.0 : val((double)v[i], absolute);",
     "const double vi = 1.0;", 2),
    ("rowdot_drops_alpha", "r = val((double)alpha, absolute) * (vi * t);", "r = vi * t;", 0),
    ("rowdot_beta_sign", "if (beta != 0.0f) r += val((double)beta, absolute) * val((double)t0[i], absolute);",
     "if (beta != 0.0f) r -= val((double)beta, absolute) * val((double)t0[i], absolute);", 0),
    ("rowdot_skips_first_entry", "for (int64_t p = row_ptr[i]; p < row_ptr[i + 1]; ++p)",
     "for (int64_t p = row_ptr[i] + 1; p < row_ptr[i + 1]; ++p)", 2),
    ("tmv_reads_u_backwards", "const double ui = val((double)u[i], absolute);",
     "const double ui = val((double)u[m - 1 - i], absolute);", 0),
    ("tmv_scatters_by_row", "S[(size_t)col_idx[p]] +=", "S[(size_t)(i % n)] +=", 1),
]


def _mutate(src: str, old: str, new: str, occurrence: int) -> str:
    pos = -1
    for _ in range(occurrence + 1):
        pos = src.find(old, pos + 1)
        assert pos >= 0, "mutation target not found: %r (occurrence %d)" % (old, occurrence)
    return src[:pos] + new + src[pos + len(old):]


@pytest.fixture(scope="module")
def mutants(tmp_path_factory):
    src = open(SRC).read()
    d = tmp_path_factory.mktemp("oracle_mutants")

    def build(mut):
        name, old, new, occ = mut
        path = d / (name + ".cpp")
        path.write_text(_mutate(src, old, new, occ))
        return name, oracle.compile_source(str(path), str(d / ("lib" + name + ".so")))

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        return dict(ex.map(build, MUTATIONS))


@pytest.mark.parametrize("mutation", [m[0] for m in MUTATIONS])
def test_pins_catch_mutant(mutants, mutation):
    lib = oracle._bind(mutants[mutation])
    caught = []
    for check in CHECKS:
        try:
            check(lib)
        except (AssertionError, oracle.OracleError) as e:
            caught.append(check.__name__)
    assert caught, "mutant %s passes every pin" % mutation
