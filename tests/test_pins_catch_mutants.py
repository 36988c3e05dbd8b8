"""The oracle's pins must fail on plausible mistakes.

Each case plants one mistake in a copy of oracle/moe_oracle.c (a dropped
term, a wrong sign or index, a transposed operand, a wrong tie rule), builds
it into a temporary library, and runs the oracle pin tests against it in a
subprocess: they must fail.  CPU only; nothing here touches the GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "int4_high_nibble_first": ("(p[i / 2] >> (4 * (int)(i % 2)))", "(p[i / 2] >> (4 * (int)(1 - i % 2)))"),
    "int4_unsigned": ("return v >= 8 ? v - 16 : v;", "return v;"),
    "int2_crumb_order": ("(p[i / 4] >> (2 * (int)(i % 4)))", "(p[i / 4] >> (2 * (int)(3 - i % 4)))"),
    "group_score_max_only": ("gscore[g] = (b < 0) ? c[a] : c[a] + c[b];", "gscore[g] = c[a];"),
    "bias_in_weights": ("      wk[j] = s[idx[j]];\n", "      wk[j] = c[idx[j]];\n"),
    "ties_to_highest": ("return va > vb || (va == vb && ia < ib);", "return va > vb || (va == vb && ia > ib);"),
    "no_scaling": ("wk[j] = wk[j] / wsum * d->routed_scaling;", "wk[j] = wk[j] / wsum;"),
    "topp_no_renormalization": ("    wsum = before;\n", "\n"),
    "topp_one_expert_short": ("while (keep < K && before < thr) before += wk[keep++];", "while (keep < K && before + wk[keep] < thr) before += wk[keep++];"),
    "int8_unsigned": ("return v >= 128 ? v - 256 : v;", "return v;"),
    "e4m3_exponent_bias": ("else v = ldexp(8.0 + (double)m, e - 10);", "else v = ldexp(8.0 + (double)m, e - 9);"),
    "requant_round_half_up": ("double v = s == 0.0f ? 0.0 : rint(w / (double)s);", "double v = s == 0.0f ? 0.0 : floor(w / (double)s + 0.5);"),
    "requant_range_8": ("const float s = (float)(m / 7.0);", "const float s = (float)(m / 8.0);"),
    "requant_block_transposed": ("const float* bs = block_scales + (r / block) * bcols;", "const float* bs = block_scales + (r % block) * 0;"),
    "sigmoid_sign": ("s[e] = 1.0 / (1.0 + exp(-z[e]));", "s[e] = 1.0 / (1.0 + exp(z[e]));"),
    "silu_sign": ("double h = g / (1.0 + exp(-g)) * u;", "double h = g / (1.0 + exp(g)) * u;"),
    "gate_up_swapped": ("double h = g / (1.0 + exp(-g)) * u;", "double h = u / (1.0 + exp(-u)) * g;"),
    "down_transposed": ("acc += weight_at(dtype, dn, dns, I, o, r) * hbuf[r];", "acc += weight_at(dtype, dn, dns, I, r % H, o % I) * hbuf[r];"),
    "no_bf16_h_rounding": ("hbuf[r] = bf16_to_double(float_to_bf16((float)hbuf[r]));", "hbuf[r] = hbuf[r];"),
    "shared_dropped": ("for (int64_t o = 0; o < H && rc == ORC_OK; ++o) out[t * H + o] += S[o];", ""),
    "combine_weight_order": ("acc += w64[t * K + j] * Y[(t * K + j) * H + o];", "acc += w64[t * K + (K - 1 - j)] * Y[(t * K + j) * H + o];"),
    "bucket_unstable": ("entries[fill[e]] = (int32_t)f;", "entries[offsets[e + 1] - 1 - (fill[e] - offsets[e])] = (int32_t)f;"),
    "logit_drop_last": ("for (int64_t h = 0; h < H; ++h)\n      acc += x_at", "for (int64_t h = 0; h < H - 1; ++h)\n      acc += x_at"),
    "rmsnorm_no_eps": ("double den = sqrt(ss / (double)hidden + eps);", "double den = sqrt(ss / (double)hidden);"),
    "softmax_wrong_ref": ("wk[j] = exp(z[idx[j]] - z0);", "wk[j] = exp(z[idx[j]] - z0) * (j + 1);"),
    "band_distance_from_lo": ("const double mid = 0.5 * ((double)lo + (double)hi);", "const double mid = (double)lo;"),
    "band_absolute_window": ("if (fabs((double)hf - mid) <= window * eb[r])", "if (fabs((double)hf - mid) <= window)"),
    "band_relative_window": ("if (fabs((double)hf - mid) <= window * eb[r])", "if (fabs((double)hf - mid) <= window * fabs((double)hf))"),
    "band_one_sided": ("if (fabs((double)hf - mid) <= window * eb[r])", "if ((double)hf - mid >= 0.0 && (double)hf - mid <= window * eb[r])"),
    "band_scale_drops_gate_term": ("ebuf[r] = fabs(dsilu * u) * ag + fabs(g * sg) * au;", "ebuf[r] = fabs(g * sg) * au;"),
    "band_scale_wrong_derivative": ("const double dsilu = sg * (1.0 + g * (1.0 - sg));", "const double dsilu = sg;"),
    "scale_of_wrong_row": ("return (double)code_at(dtype, row, c) * (double)scale[r];", "return (double)code_at(dtype, row, c) * (double)scale[r ^ 1];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_fail_on_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mut = tmp_path / "moe_oracle.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-shared",
                    "-fPIC", "-I", os.path.join(ROOT, "oracle"), str(mut), "-o", str(lib), "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, MOE_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    tests = [os.path.join(ROOT, "tests", f) for f in sorted(os.listdir(os.path.join(ROOT, "tests")))
             if f.startswith("test_oracle_")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
