"""Planted mistakes in copies of the oracle must each fail a pin (CPU only).

Each mutant is the oracle's C source with one plausible mistake put in by a
text substitution (a dropped term, a wrong sign, a wrong index, a
transposed operand, an off-by-one mask), built with gcc into a temporary
directory.  The real oracle source is never modified.  A mutant that passes
every pin would mean the pins leave that part of the oracle unchecked.
"""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

MUTANTS = {
    "no_max_subtraction": ("p[j] = exp(x[j] - m);", "p[j] = exp(x[j]);"),
    "mask_off_by_one": ("if (causal && j > i) {", "if (causal && j >= i && j > 0) {"),
    "mask_dropped": ("if (causal && j > i) {", "if (0) {"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "lse_without_max": ("lse[i] = m + log(l);", "lse[i] = log(l);"),
    "lse_log2": ("lse[i] = m + log(l);", "lse[i] = m + log2(l);"),
    "pv_wrong_row": ("const double* vj = v + j * d;\n      for (int64_t c = 0; c < d; ++c) oi[c]",
                     "const double* vj = v + i * d;\n      for (int64_t c = 0; c < d; ++c) oi[c]"),
    "no_normalisation": ("for (int64_t j = 0; j < n; ++j) p[j] = p[j] / l;", ""),
    "ds_sign": ("dS[i * N + j] = P[i * N + j] * (dp - D[i]);", "dS[i * N + j] = P[i * N + j] * (dp + D[i]);"),
    "ds_no_D": ("dS[i * N + j] = P[i * N + j] * (dp - D[i]);", "dS[i * N + j] = P[i * N + j] * dp;"),
    "dq_no_scale": ("    for (int64_t c = 0; c < d; ++c) dq[i * d + c] *= scale;\n", ""),
    "dk_transposed": ("const double g = dS[i * N + j];\n      const double pij",
                      "const double g = dS[j * N + i];\n      const double pij"),
    "dv_uses_dS": ("dv[j * d + c] += pij * dout[i * d + c];", "dv[j * d + c] += g * dout[i * d + c];"),
    "D_uses_V": ("acc += dout[i * d + c] * O[i * d + c];", "acc += dout[i * d + c] * v[i * d + c];"),
    "dq_uses_V": ("dq[i * d + c] += g * k[j * d + c];", "dq[i * d + c] += g * v[j * d + c];"),
    "rows_wrong_index": ("const int64_t i = rows[r];", "const int64_t i = r;"),
    "rect_mask_unshifted": ("if (causal && j > i + offset) {", "if (causal && j > i) {"),
    "rect_scale_dropped": ("s[j] = dot * scale;", "s[j] = dot;"),
    "rect_lse_log2": ("lse[i] = log(l) + m;", "lse[i] = log2(l) + m;"),
    "rect_pv_key_offset": ("oi[c] += p[j] * vj[c];", "oi[c] += p[j] * vj[c] * (j + 1 < Nk);"),
    "rect_bwd_mask_unshifted": ("if (causal && t > r + shift) {", "if (causal && t > r) {"),
    "rect_bwd_ds_sign": ("dSr[r * Nk + t] = Pr[r * Nk + t] * (dpr - Dr[r]);",
                         "dSr[r * Nk + t] = Pr[r * Nk + t] * (dpr + Dr[r]);"),
    "rect_bwd_dk_uses_P": ("ak += dSr[r * Nk + t] * q[r * d + c];", "ak += Pr[r * Nk + t] * q[r * d + c];"),
    "rect_bwd_dv_uses_V": ("av += Pr[r * Nk + t] * dout[r * d + c];", "av += Pr[r * Nk + t] * v[t * d + c];"),
    "rect_bwd_dq_no_scale": ("dq[r * d + c] = scale * acc;", "dq[r * d + c] = acc;"),
    "rect_bwd_D_uses_Q": ("dd += dout[r * d + c] * Or[r * d + c];", "dd += dout[r * d + c] * q[r * d + c];"),
    "rect_bwd_dk_wrong_key": ("ak += dSr[r * Nk + t] * q[r * d + c];", "ak += dSr[r * Nk + (Nk - 1 - t)] * q[r * d + c];"),
    "dq_rows_D_from_dO": ("Di += doi[c] * orow[c];", "Di += doi[c] * doi[c];"),
    "dq_rows_no_scale": ("for (int64_t c = 0; c < d; ++c) dqi[c] *= scale;", ""),
    "dq_rows_uses_v": ("dqi[c] += dst * k[t * d + c];", "dqi[c] += dst * v[t * d + c];"),
    "e4m3_bias": ("ldexp(8.0 + m, e - 10)", "ldexp(8.0 + m, e - 11)"),
    "e4m3_subnormal_as_normal": ("(e == 0) ? ldexp((double)m, -9) :", ""),
    "e4m3_no_sign": ("return sign ? -mag : mag;", "return mag;"),
    "mx_block_of_16": ("scales[r * nb + c / 32]", "scales[r * nb + c / 16 % nb]"),
    "e8m0_bias": ("ldexp(1.0, (int)e - 127)", "ldexp(1.0, (int)e - 128)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / f"mut_{name}.c"
    mut.write_text(src.replace(old, new))
    so = str(tmp_path / f"libmut_{name}.so")
    oracle.build(str(mut), so)
    lib = oracle.load(so)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, FloatingPointError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
