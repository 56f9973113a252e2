"""The pins have teeth: plant one plausible mistake at a time in a copy of the
oracle's C source (on the CPU, in a temporary directory), build it, run the
whole pin battery against that build in a child process, and require that at
least one pin fails (or the build crashes).  The real oracle is never touched.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("share_without_current_bid", "(D[j] + p[j] + eps)", "(D[j] + eps)"),
    ("committed_inclusive", "(D[j] + p[j] + eps)", "(D[j] + 2.0 * p[j] + eps)"),
    ("eps_dropped", "(D[j] + p[j] + eps)", "(D[j] + p[j])"),
    ("tau_ignored", "const double c = tau / sqrt((double)d);",
     "const double c = 1.0 / sqrt((double)d);"),
    ("no_sqrt_d", "const double c = tau / sqrt((double)d);", "const double c = tau;"),
    ("diagonal_key_hidden", "const long lo = (long)(i + 1) * t / n, hi = (long)(i + 1) * (t + 1) / n;",
     "const long lo = (long)(i) * t / n, hi = (long)(i) * (t + 1) / n;"),
    ("bids_not_normalised", "p[j] = exp(p[j] - l);", "p[j] = exp(p[j] - M);"),
    ("lse_wrong_sign", "const double l = M + log(Z);", "const double l = M - log(Z);"),
    ("diagonal_bid_not_committed", "        D[j] += p[j];", "        if (i > j) D[j] += p[j];"),
    ("demand_never_committed", "        D[j] += p[j];\n", "\n"),
    ("shares_not_renormalised", "Oh[(size_t)li * d + e] = acc[e] / r;",
     "Oh[(size_t)li * d + e] = acc[e];"),
    ("value_rows_reversed",
     "          for (int e = 0; e < d; ++e) acc[e] += share * Vh[(size_t)j * d + e];",
     "          for (int e = 0; e < d; ++e) acc[e] += share * Vh[(size_t)(i - j) * d + e];"),
    ("tempered_value_row_off_by_one", "acc[e] += p[j] * Vh[(size_t)j * d + e];",
     "acc[e] += p[j] * Vh[(size_t)(j > 0 ? j - 1 : 0) * d + e];"),
    ("decode_committed_inclusive", "(Dh[j] + p[j] + eps)", "(Dh[j] + 2.0 * p[j] + eps)"),
    ("decode_first_key_not_updated", "for (int j = 0; j < L; ++j) Dh[j] += p[j];",
     "for (int j = 1; j < L; ++j) Dh[j] += p[j];"),
    ("decode_updates_with_share", "for (int j = 0; j < L; ++j) Dh[j] += p[j];",
     "for (int j = 0; j < L; ++j) Dh[j] += p[j] / (Dh[j] + p[j] + eps);"),
    ("bf16_widening_shift", "<< 16;", "<< 15;"),
    ("yarn_coefficient", "return 0.1 * log(s) + 1.0;", "return 0.1 * log2(s) + 1.0;"),
    ("prefill_demand_in_ignored",
     "if (demand) memcpy(D, demand + (size_t)bh * Lcap, sizeof(double) * (size_t)Tk);", ""),
    ("prefill_keys_from_chunk_start",
     "causal_bids(Qh + (size_t)li * d, Kh, i, d, c, p, 0)",
     "causal_bids(Qh + (size_t)li * d, Kh, li, d, c, p, 0)"),
    ("prefill_cache_stride", "kbase = (size_t)bh * Lcap * d", "kbase = (size_t)bh * Tk * d"),
    ("prefill_tempered_keys_from_chunk_start",
     "causal_bids(Qh + (size_t)(i - P) * d, Kh, i, d, c, p, inner)",
     "causal_bids(Qh + (size_t)(i - P) * d, Kh, i - P, d, c, p, inner)"),
    ("bwd_dtau_without_sqrt_d", "dtau[bh] = acc / sqrt((double)d);", "dtau[bh] = acc;"),
    ("bwd_dtau_from_bids", "acc += dP[(size_t)i * T + j] * dot(Q + (size_t)i * d, K + (size_t)j * d, d);",
     "acc += P[(size_t)i * T + j] * dot(Q + (size_t)i * d, K + (size_t)j * d, d);"),
    ("bwd_suffix_exclusive",
     "          col[j] += dPi[j] * Pi[j] / (Di[j] * Di[j]);\n          dPi[j] = dPi[j] / Di[j] - col[j];",
     "          dPi[j] = dPi[j] / Di[j] - col[j];\n          col[j] += dPi[j] * Pi[j] / (Di[j] * Di[j]);"),
    ("bwd_later_rows_ignored", "dPi[j] = dPi[j] / Di[j] - col[j];",
     "dPi[j] = dPi[j] / Di[j] - dPi[j] * Pi[j] / (Di[j] * Di[j]);"),
    ("bwd_delta_dropped", "dPi[j] = (dPi[j] - delta) / r[i];", "dPi[j] = dPi[j] / r[i];"),
    ("bwd_softmax_rho_dropped", "dPi[j] = Pi[j] * (dPi[j] - rho);", "dPi[j] = Pi[j] * dPi[j];"),
    ("bwd_dk_from_k", "dkj[e] += c * s * Q[(size_t)i * d + e];",
     "dkj[e] += c * s * K[(size_t)i * d + e];"),
    ("bwd_dv_from_bids", "dvj[e] += a * dO[(size_t)i * d + e];",
     "dvj[e] += P[(size_t)i * T + j] * dO[(size_t)i * d + e];"),
    ("bwd_per_head_tau_ignored", "(tau_bh ? tau_bh[bh] : tau) / sqrt((double)d)",
     "tau / sqrt((double)d)"),
    ("rope_turns_clockwise",
     "      out[(size_t)r * d + 2 * m] = a * c - b * sn;\n      out[(size_t)r * d + 2 * m + 1] = a * sn + b * c;",
     "      out[(size_t)r * d + 2 * m] = a * c + b * sn;\n      out[(size_t)r * d + 2 * m + 1] = -a * sn + b * c;"),
    ("rope_position_offset_ignored",
     "const double theta = (double)(pos0 + t) * freq[m];",
     "const double theta = (double)t * freq[m];"),
    ("rope_half_split_pairs",
     "      const double a = widen(x, dtype, (size_t)r * d + 2 * m);\n      const double b = widen(x, dtype, (size_t)r * d + 2 * m + 1);\n      out[(size_t)r * d + 2 * m] = a * c - b * sn;\n      out[(size_t)r * d + 2 * m + 1] = a * sn + b * c;",
     "      const double a = widen(x, dtype, (size_t)r * d + m);\n      const double b = widen(x, dtype, (size_t)r * d + m + d / 2);\n      out[(size_t)r * d + m] = a * c - b * sn;\n      out[(size_t)r * d + m + d / 2] = a * sn + b * c;"),
    ("rope_bf16_seven_bits", "const double scaled = ldexp(m, 8);", "const double scaled = ldexp(m, 7);"),
    ("rope_bf16_ties_up", "if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;",
     "if (frac >= 0.5) r += 1.0;"),
]

RUNNER = r"""
import sys, traceback
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
oracle.use_library(oracle.load_library({lib!r}))
import pins
failed = []
for pin in pins.ALL_PINS:
    try:
        pin()
    except Exception:
        failed.append(pin.__name__)
print("FAILED_PINS", len(failed), " ".join(failed))
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    import oracle

    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new)
    with tempfile.TemporaryDirectory() as tmp:
        msrc = os.path.join(tmp, "oracle_mutant.c")
        mlib = os.path.join(tmp, "liboracle_mutant.so")
        with open(msrc, "w") as f:
            f.write(mutated)
        oracle.build(msrc, mlib)
        r = subprocess.run([sys.executable, "-c", RUNNER.format(
            root=ROOT, tests=os.path.join(ROOT, "tests"), lib=mlib)],
            capture_output=True, text=True, timeout=300,
            env={**os.environ, "OMP_NUM_THREADS": "4"})
    if r.returncode != 0:
        return  # the planted mistake crashed the battery: caught
    line = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED_PINS")]
    assert line, r.stdout + r.stderr
    assert int(line[0].split()[1]) >= 1, f"no pin caught mutant {name}"
