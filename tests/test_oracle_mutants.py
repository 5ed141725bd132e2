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
     "double dk = sq_dist(v, book + (int64_t)k * dim, dim);",
     "double dk = sq_dist(v, book + (int64_t)k, dim);"),
    ("residual subtracts the wrong row",
     "const float *c = book + (int64_t)k1 * jb->dim;", "const float *c = book + (int64_t)k1;"),
    ("second-best not shifted on a new best",
     "            d2 = d1;\n", ""),
    ("best and second swapped in the report",
     "if (jb->best) jb->best[n * jb->n_stages + q] = d1;",
     "if (jb->best) jb->best[n * jb->n_stages + q] = d2;"),
    ("first codeword never compared",
     "double d1 = sq_dist(v, book, dim);", "double d1 = INFINITY;"),
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
     "if (b) s = s + (double)b[o];", ""),
    ("linear uses the transposed weight",
     "for (int32_t i = 0; i < in_dim; ++i) s = s + (double)v[i] * (double)wo[i];",
     "for (int32_t i = 0; i < in_dim; ++i) s = s + (double)v[i] * (double)w[(int64_t)i * out_dim + o];"),
    ("linear accumulates in float32",
     "double s = 0.0;\n        for (int32_t i = 0; i < in_dim; ++i)",
     "float s = 0.0f;\n        for (int32_t i = 0; i < in_dim; ++i)"),
    ("projected: every stage projects with stage 0's W_in",
     "linear_row(jb->w_in + (int64_t)q * dim * hid, b_in, r, hid, dim, e);",
     "linear_row(jb->w_in, b_in, r, hid, dim, e);"),
    ("projected: b_in dropped",
     "const float *b_in = jb->b_in ? jb->b_in + (int64_t)q * dim : NULL;",
     "const float *b_in = NULL;"),
    ("projected: given encodings ignored",
     "const float *pick_on = jb->e_given ? jb->e_given + at : e;",
     "const float *pick_on = e;"),
    ("projected: encodings reported frame-major",
     "const int64_t at = ((int64_t)q * jb->n_frames + n) * dim;",
     "const int64_t at = (n * jb->n_stages + q) * dim;"),
    ("projected: every stage searches codebook 0",
     "const float *stage_book = jb->books + (int64_t)q * jb->n_codes * dim;",
     "const float *stage_book = jb->books;"),
    ("projected: out-projection with stage 0's W_out",
     "linear_row(jb->w_out + (int64_t)q * hid * dim, b_out, stage_book + (int64_t)k1 * dim, dim, hid, p);",
     "linear_row(jb->w_out, b_out, stage_book + (int64_t)k1 * dim, dim, hid, p);"),
    ("projected: out-projection of the wrong codeword row",
     "linear_row(jb->w_out + (int64_t)q * hid * dim, b_out, stage_book + (int64_t)k1 * dim, dim, hid, p);",
     "linear_row(jb->w_out + (int64_t)q * hid * dim, b_out, stage_book + (int64_t)k1, dim, hid, p);"),
    ("projected: residual adds the projected codeword",
     "for (int32_t i = 0; i < hid; ++i) r[i] = (float)(r[i] - p[i]);",
     "for (int32_t i = 0; i < hid; ++i) r[i] = (float)(r[i] + p[i]);"),
    ("projected: b_out dropped in the encode",
     "const float *b_out = jb->b_out ? jb->b_out + (int64_t)q * hid : NULL;\n            linear_row(jb->w_out + (int64_t)q * hid * dim, b_out, stage_book",
     "const float *b_out = NULL;\n            linear_row(jb->w_out + (int64_t)q * hid * dim, b_out, stage_book"),
    ("projected decode: b_out dropped",
     "const float *b_out = jb->b_out ? jb->b_out + (int64_t)q * hid : NULL;\n            linear_row(jb->w_out + (int64_t)q * hid * dim, b_out,\n",
     "const float *b_out = NULL;\n            linear_row(jb->w_out + (int64_t)q * hid * dim, b_out,\n"),
    ("projected decode: stage q's code looked up in codebook 0",
     "jb->books + ((int64_t)q * jb->n_codes + code) * dim, dim, hid, p);",
     "jb->books + ((int64_t)0 * jb->n_codes + code) * dim, dim, hid, p);"),
    ("projected decode: stage order reversed",
     "            int32_t code = jb->codes[n * jb->codes_ld + q];",
     "            int32_t code = jb->codes[n * jb->codes_ld + (jb->n_stages - 1 - q)];"),
    ("cosine: the encoding is not normalized",
     "                unit_vector(pick_on, dim, u);\n",
     "                for (int32_t j = 0; j < dim; ++j) u[j] = pick_on[j];\n"),
    ("cosine: codewords are not normalized",
     "for (int64_t k = 0; k < rows; ++k) unit_vector(books + k * dim, dim, units + k * dim);",
     "for (int64_t k = 0; k < rows * dim; ++k) units[k] = books[k];"),
    ("cosine: no norm floor",
     "    if (norm < 1e-12) norm = 1e-12;\n", ""),
    ("cosine: every stage searches normalized codebook 0",
     "k1 = nearest_unit(u, jb->units + (int64_t)q * jb->n_codes * dim, jb->n_codes, dim, &d1, &d2);",
     "k1 = nearest_unit(u, jb->units, jb->n_codes, dim, &d1, &d2);"),
    ("cosine: ties go to the highest index",
     "        if (acc < lo) {", "        if (acc <= lo) {"),
    ("cosine: norm without the square root",
     "double norm = sqrt(ss);", "double norm = ss;"),
    ("projected decode: bad codes read row 0",
     "                for (int32_t i = 0; i < hid; ++i) acc[i] = NAN;\n                break;",
     "                code = 0;"),
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
