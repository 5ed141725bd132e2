"""Planted mistakes in the CPU oracle must each fail at least one pin (no GPU).

Every mutant is a copy of ``oracle/rvq_oracle.c`` with one plausible slip
(a wrong sign, index, stride or comparison, a dropped term, a transposed
operand) compiled into a temporary directory. The pins in
``oracle_pins.py`` are run against it; a mutant that passes them all would
mean the pins cannot see that slip.
"""

import os

import pytest

import oracle
import oracle_pins

MUTANTS = [
    ("ties go to the highest index",
     "if (dk < d1) {", "if (dk <= d1) {"),
    ("residual update adds the codeword",
     "r[j] = (float)(r[j] - c[j]);", "r[j] = (float)(r[j] + c[j]);"),
    ("residual never updated",
     "for (int32_t j = 0; j < jb->dim; ++j) r[j] = (float)(r[j] - c[j]);", ""),
    ("every stage searches codebook 0",
     "const float *book = jb->books + (int64_t)q * jb->n_codes * jb->dim;",
     "const float *book = jb->books;"),
    ("distance drops the square",
     "s = s + t * t;", "s = s + fabs(t);"),
    ("distance with a wrong sign",
     "double t = (double)r[j] - (double)c[j];", "double t = (double)r[j] + (double)c[j];"),
    ("transposed codebook row stride",
     "double dk = sq_dist(r, book + (int64_t)k * jb->dim, jb->dim);",
     "double dk = sq_dist(r, book + (int64_t)k, jb->dim);"),
    ("residual subtracts the wrong row",
     "const float *c = book + (int64_t)k1 * jb->dim;", "const float *c = book + (int64_t)k1;"),
    ("second-best not shifted on a new best",
     "                    d2 = d1;\n", ""),
    ("best and second swapped in the report",
     "if (jb->best) jb->best[n * jb->n_stages + q] = d1;",
     "if (jb->best) jb->best[n * jb->n_stages + q] = d2;"),
    ("first codeword never compared",
     "double d1 = sq_dist(r, book, jb->dim);", "double d1 = INFINITY;"),
    ("decode stage order reversed",
     "            int32_t k = jb->codes[n * jb->codes_ld + q];\n"
     "            if (k < 0 || k >= jb->n_codes) {",
     "            int32_t qq = jb->n_stages - 1 - q;\n"
     "            int32_t k = jb->codes[n * jb->codes_ld + qq];\n"
     "            if (k < 0 || k >= jb->n_codes) {"),
    ("decode reads stage q's code from stage 0",
     "const float *c = jb->books + ((int64_t)q * jb->n_codes + k) * jb->dim;",
     "const float *c = jb->books + ((int64_t)0 * jb->n_codes + k) * jb->dim;"),
    ("decode ignores bad codes",
     "                for (int32_t j = 0; j < jb->dim; ++j) o[j] = NAN;\n                break;",
     "                k = 0;"),
    ("linear drops the bias",
     "if (jb->b) s = s + (double)jb->b[o];", ""),
    ("linear uses the transposed weight",
     "for (int32_t i = 0; i < jb->in_dim; ++i) s = s + (double)hn[i] * (double)wo[i];",
     "for (int32_t i = 0; i < jb->in_dim; ++i) s = s + (double)hn[i] * (double)jb->w[(int64_t)i * jb->out_dim + o];"),
    ("linear accumulates in float32",
     "double s = 0.0;\n            for (int32_t i = 0; i < jb->in_dim; ++i)",
     "float s = 0.0f;\n            for (int32_t i = 0; i < jb->in_dim; ++i)"),
]



@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for '{name}' must occur exactly once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(str(path), str(tmp_path / "libmutant.so"), werror=False)
    o = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin notices the planted mistake: {name}"


def test_unmutated_copy_passes_all_pins(tmp_path):
    """Control: the same build route with no mutation passes every pin."""
    lib = oracle.build(oracle.SOURCE, str(tmp_path / "libcopy.so"))
    o = oracle.Oracle(lib)
    for pin in oracle_pins.ALL_PINS:
        pin(o)
    assert os.path.exists(lib)
