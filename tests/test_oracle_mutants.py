"""Planted mistakes in copies of the oracle must each fail at least one pin (CPU only).

Each mutant is a one-line edit of ``oracle/oracle.cpp``: a dropped term, a wrong
sign, a wrong index, a transposed operand, a wrong constant, a missing swap. The
copy is compiled into a temporary directory and the whole pin battery is run on
it; the test passes when some pin rejects it. This shows that the pins would
catch the plausible mistakes they are meant to catch.
"""

import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "drop_west": ("T t = (w + e) + (s + n);", "T t = (e + e) + (s + n);"),
    "drop_north": ("T t = (w + e) + (s + n);", "T t = (w + e) + (s + s);"),
    "source_sign": ("if (b) t = t + b[at(nx, i, j)];\n            B[", "if (b) t = t - b[at(nx, i, j)];\n            B["),
    "source_dropped": ("if (b) t = t + b[at(nx, i, j)];\n            B[", "if (b) t = t;\n            B["),
    "source_h_not_squared": ("const double hh = h * h;", "const double hh = h;"),
    "east_index": ("const T e = A[at(nx, i, j + 1)];", "const T e = A[at(nx, i, j)];"),
    "south_row": ("const T s = A[at(nx, i - 1, j)];", "const T s = A[at(nx, i - 1, j - 1)];"),
    "transposed_store": ("B[at(nx, i, j)] = T(0.25) * t;", "B[at(nx, j % ny, i % nx)] = T(0.25) * t;"),
    "weight": ("B[at(nx, i, j)] = T(0.25) * t;", "B[at(nx, i, j)] = T(0.2) * t;"),
    "no_swap": ("A.swap(B);", "(void)0;"),
    "gauss_seidel_in_place": ("sweep<T>(nx, ny, A.data(), B.data(), bp);",
                              "sweep<T>(nx, ny, A.data(), A.data(), bp);"),
    "ring_overwritten": ("for (int j = 1; j <= nx - 2; ++j) {\n            const T w",
                         "for (int j = 1; j <= nx - 1; ++j) {\n            const T w"),
    "residual_centre_weight": ("const double r = t - 4.0 * static_cast<double>(A[at(nx, i, j)]);",
                               "const double r = t - 2.0 * static_cast<double>(A[at(nx, i, j)]);"),
    "residual_source_sign": ("if (b) t = t + static_cast<double>(b[at(nx, i, j)]);",
                             "if (b) t = t - static_cast<double>(b[at(nx, i, j)]);"),
    "residual_not_sqrt": ("return std::sqrt(acc);", "return acc;"),
    # red-black Gauss-Seidel
    "rb_black_first": ("rb_half<T>(nx, ny, U.data(), bp, 0);  // red: i + j even\n        rb_half<T>(nx, ny, U.data(), bp, 1);",
                       "rb_half<T>(nx, ny, U.data(), bp, 1);  // red: i + j even\n        rb_half<T>(nx, ny, U.data(), bp, 0);"),
    "rb_black_skipped": ("rb_half<T>(nx, ny, U.data(), bp, 1);  // black", "(void)0;  // black"),
    "rb_row_parity": ("if (((i + j) & 1) != parity) continue;", "if ((i & 1) != parity) continue;"),
    "rb_east_index": ("const T east = U[at(nx, i, j + 1)];", "const T east = U[at(nx, i, j)];"),
    "rb_south_row": ("const T south = U[at(nx, i - 1, j)];", "const T south = U[at(nx, i - 1, j - 1)];"),
    "rb_source_sign": ("if (b) t = t + b[at(nx, i, j)];\n            U[", "if (b) t = t - b[at(nx, i, j)];\n            U["),
    "rb_weight": ("U[at(nx, i, j)] = T(0.25) * t;", "U[at(nx, i, j)] = T(0.2) * t;"),
    "rb_jacobi_instead": ("rb_half<T>(nx, ny, U.data(), bp, 0);  // red: i + j even\n        rb_half<T>(nx, ny, U.data(), bp, 1);",
                          "{ std::vector<T> V(U); sweep<T>(nx, ny, V.data(), U.data(), bp); }"),
    "two_sweeps_per_step": ("if (k == K) break;\n        sweep<T>", "if (k == K) break;\n        sweep<T>(nx, ny, A.data(), B.data(), bp);\n        A.swap(B);\n        sweep<T>"),
}


def _run_battery(orc):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
        except (ValueError, OverflowError, ZeroDivisionError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = oracle.compile_copy(src.replace(old, new), os.path.join(str(tmp_path), f"lib_{name}.so"))
    failed = _run_battery(oracle.Oracle(path))
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    path = oracle.compile_copy(oracle.source_text(), os.path.join(str(tmp_path), "lib_same.so"))
    assert _run_battery(oracle.Oracle(path)) == []
