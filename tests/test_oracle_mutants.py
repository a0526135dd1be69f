"""Plant plausible mistakes in a copy of the oracle's C source, build each on
the CPU, and require that every mutant fails at least one pin.  This shows
the pins constrain every part of the oracle (scale, sign, index, mask,
normalisation, recurrence), not just that the oracle passes them."""
import os

import numpy as np
import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("dS_sign", "row[j] = P[i * Nk + j] * (row[j] - r);", "row[j] = P[i * Nk + j] * (row[j] + r);"),
    ("r_without_P", "r += P[i * Nk + j] * row[j];", "r += row[j];"),
    ("dQ_no_scale", "g[c] *= scale;", "g[c] *= 1.0;"),
    ("dK_no_scale", "a[c] *= scale;", "a[c] *= 1.0;"),
    ("dQ_uses_V", "g[c] += w * k[j * d + c];", "g[c] += w * v[j * d + c];"),
    ("dK_uses_P", "ws = dS[i * Nk + j], wp", "ws = P[i * Nk + j], wp"),
    ("dV_uses_dS", "wp = Pv[i * Nk + j];", "wp = dS[i * Nk + j];"),
    ("dV_uses_Q", "b[c] += wp * go[i * d + c];", "b[c] += wp * q[i * d + c];"),
    ("mask_reversed", "return !causal || j <= i;", "return !causal || j >= i;"),
    ("mask_strict", "return !causal || j <= i;", "return !causal || j < i || j == 0;"),
    ("no_scale_in_S", "row[j] = scale * dot(Q + i * d, K + j * d, d);", "row[j] = dot(Q + i * d, K + j * d, d);"),
    ("sum_without_shift", "if (allowed(i, j, causal)) l += exp(row[j] - m);", "if (allowed(i, j, causal)) l += exp(row[j]);"),
    ("lse_sign", "LSE[i] = m + log(l);", "LSE[i] = m - log(l);"),
    ("online_l_old_unweighted", "*l1 = w_old * *l1 + w_new * l2;", "*l1 = *l1 + w_new * l2;"),
    ("online_u_old_unweighted", "u1[c] = w_old * u1[c] + w_new * u2[c];", "u1[c] = u1[c] + w_new * u2[c];"),
    ("online_weight_sign", "const double w_old = exp(*m1 - m), w_new = exp(m2 - m);",
     "const double w_old = exp(m - *m1), w_new = exp(m - m2);"),
    ("online_tile_unshifted", "const double w = exp(s[j] - mx);", "const double w = exp(s[j]);"),
    ("online_max_not_kept", "    *m1 = m;\n}", "    *m1 = m2;\n}"),
    ("rows_no_mask", "if (!allowed(i, j, causal)) continue;\n                const double p", "const double p"),
    ("philox_key_not_bumped", "            k1 += kPhiloxWeyl1;\n", "            k1 += 0u;\n"),
    ("philox_hi_for_lo", "        c1 = lo1;", "        c1 = hi1;"),
    ("dropout_keep_strict", "keep[(h * Nq + i) * Nk + j] = byte >= (uint32_t)t;",
     "keep[(h * Nq + i) * Nk + j] = byte > (uint32_t)t;"),
    ("dropout_word_by_key", "(w[i % 4] >> (8 * (j % 4)))", "(w[j % 4] >> (8 * (j % 4)))"),
    ("dropout_counter_no_head", "(uint32_t)(i / 4), (uint32_t)(bh0 + h), 0u}", "(uint32_t)(i / 4), 0u, 0u}"),
    ("dropout_fwd_no_keep_scale", "P[e] = z[e] ? P[e] * keep_scale : 0.0;", "P[e] = z[e] ? P[e] : 0.0;"),
    ("dropout_dP_no_keep_scale", "(z[i * Nk + j] ? g * keep_scale : 0.0)", "(z[i * Nk + j] ? g : 0.0)"),
    ("dropout_dV_undropped", "scale, P, Pd, z, keep_scale,", "scale, P, P, z, keep_scale,"),
    ("dropout_r_with_dropped_P", "r += P[i * Nk + j] * row[j];", "r += Pv[i * Nk + j] * row[j];"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, (name, src.count(old))
    mutant = tmp_path / ("oracle_%s.c" % name)
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / ("liboracle_%s.so" % name)
    oracle.compile_source(str(mutant), str(lib))
    return oracle.Oracle(str(lib))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    o = _build_mutant(tmp_path, name, old, new)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(divide="raise", invalid="raise"):  # a NaN or division by zero is a catch too
                pin(o)
        except (AssertionError, FloatingPointError, RuntimeError, ValueError, ZeroDivisionError):
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
