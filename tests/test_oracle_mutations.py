"""Planted mistakes in a copy of the oracle must each fail at least one pin (CPU only).

Each mutation is a plausible slip in oracle.c (a dropped term, a wrong sign, a wrong
index or chunk count, a transposed operand, an exponent-bias slip in a decoder, an
off-by-one in segment lookup). The copy is compiled to a temporary library; the
real oracle is untouched.
"""

import os
import subprocess

import pytest

import oracle
from test_oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "drop_y0": ("yr[n] = J->dec(y0row[n]) + s * acc;", "yr[n] = s * acc;"),
    "sign": ("yr[n] = J->dec(y0row[n]) + s * acc;", "yr[n] = J->dec(y0row[n]) - s * acc;"),
    "drop_scale": ("yr[n] = J->dec(y0row[n]) + s * acc;", "yr[n] = J->dec(y0row[n]) + acc;"),
    "page_index_off_by_one": ("int64_t entry = first + (int64_t)row * c + e / J->P;",
                              "int64_t entry = first + (int64_t)row * c + (e + 1) / J->P;"),
    "page_offset": ("return J->pool + page * (int64_t)J->P + e % J->P;",
                    "return J->pool + page * (int64_t)J->P + (e + 1) % J->P;"),
    "b_block_start": ("const int64_t baseB = J->base[i] + (int64_t)r * cA;",
                      "const int64_t baseB = J->base[i] + (int64_t)r * cB;"),
    "b_chunks_transposed": ("paged_elem(J, baseB, k, cB, n)", "paged_elem(J, baseB, k, cA, n)"),
    "a_row_from_b": ("paged_elem(J, baseA, k, cA, j)", "paged_elem(J, baseB, k, cB, j % J->d_out)"),
    "shrink_uses_y0": ("acc += J->dec(xrow[j]) * J->dec(*a);",
                       "acc += J->dec(y0row[j % J->d_out]) * J->dec(*a);"),
    "expand_rank_short": ("for (int32_t k = 0; k < r; ++k) {\n        const uint16_t* b",
                          "for (int32_t k = 1; k < r; ++k) {\n        const uint16_t* b"),
    "f16_bias": ("v = ldexp((double)(fr | 0x400), ex - 25);", "v = ldexp((double)(fr | 0x400), ex - 24);"),
    "f16_subnormal": ("v = ldexp((double)fr, -24);", "v = ldexp((double)fr, -25);"),
    "bf16_bias": ("v = ldexp((double)(fr | 0x80), ex - 134);", "v = ldexp((double)(fr | 0x80), ex - 133);"),
    "segment_lookup": ("if (t >= seg_offsets[s] && t < seg_offsets[s + 1]) return seg_adapter[s];",
                       "if (t >= seg_offsets[s] && t <= seg_offsets[s + 1]) return seg_adapter[s];"),
    "decode_token_offset": ("return token_adapter[t - seg_end];", "return token_adapter[t - seg_end + (seg_end > 0)];"),
    "rank0_not_idle": ("if (r == 0) {", "if (r < 0) {"),
    "shrink_rank_short": ("for (int32_t k = 0; k < r; ++k) {\n      double acc = 0.0;\n      for (int32_t j",
                          "for (int32_t k = 0; k < r - 1; ++k) {\n      double acc = 0.0;\n      for (int32_t j"),
    "shrink_d_in_short": ("for (int32_t j = 0; j < J->d_in; ++j) {", "for (int32_t j = 0; j < J->d_in - 1; ++j) {"),
    "expand_d_out_short": ("for (int32_t n = 0; n < J->d_out; ++n) {\n      double acc",
                           "for (int32_t n = 0; n < J->d_out - 1; ++n) {\n      double acc"),
    # the previous token's row (stays inside the buffers)
    "x_row_of_other_token": ("const uint16_t* xrow = J->x + t * (int64_t)J->d_in;",
                             "const uint16_t* xrow = J->x + (t > 0 ? t - 1 : t) * (int64_t)J->d_in;"),
    "y0_row_of_other_token": ("const uint16_t* y0row = J->y0 + t * (int64_t)J->d_out;",
                              "const uint16_t* y0row = J->y0 + (t > 0 ? t - 1 : t) * (int64_t)J->d_out;"),
    "scale_of_adapter_0": ("const double s = J->scale[i];", "const double s = J->scale[0];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    so = str(tmp_path / "liboracle_mutant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                    str(mutant), "-o", so, "-lm"], check=True)
    lib = oracle.load(so)
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, oracle.OracleError):
            caught.append(pin.__name__)
    assert caught, f"mutation {name} passed every pin"
