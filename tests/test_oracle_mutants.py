"""The reference's pins must catch plausible mistakes.  Each case plants one
mistake in a private copy of the reference's C source (on the CPU), compiles
it, and runs the pin suite against that copy: the suite has to fail."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "cpattn_oracle.c")

MUTANTS = {
    "causal_drops_diagonal": ("if (kind == OR_CAUSAL) return xk <= xq;",
                              "if (kind == OR_CAUSAL) return xk < xq;"),
    "tree_sees_own_future": ("if (sq == sk) return xk <= xq;", "if (sq == sk) return 1;"),
    "tree_sees_siblings": ("return is_strict_ancestor(parent, n_seg, sk, sq);",
                           "return sk < sq;"),
    "merge_weight_sign": ("double a = exp(la - m), b = exp(lb - m);",
                          "double a = exp(m - la), b = exp(m - lb);"),
    "lse_drops_max": ("double lse = m + log(z);", "double lse = log(z);"),
    "key_operand_swapped": ("                           widen(K, dtype, h * k_sh + j * k_st + c);",
                            "                           widen(V, dtype, h * v_sh + j * v_st + c);"),
    "scale_dropped": ("s[a] = acc * scale;", "s[a] = acc;"),
    "output_unnormalised": ("double p = exp(s[a] - lse);", "double p = exp(s[a] - m);"),
    "window_off_by_one": ("if (lq - lk >= window) continue;", "if (lq - lk > window) continue;"),
    "window_on_storage_positions": ("int64_t lq = lp ? lp[qpos[i]] : qpos[i], lk = lp ? lp[kpos[j]] : kpos[j];",
                                    "int64_t lq = qpos[i], lk = kpos[j];"),
    "backward_drops_D": ("double ds = p * (gv - D);", "double ds = p * gv;"),
    "backward_dk_from_k": ("dK[(h * nk + j) * d + c] += scale * ds * widen(Q, dtype, h * q_sh + i * q_st + c);",
                           "dK[(h * nk + j) * d + c] += scale * ds * widen(K, dtype, h * k_sh + j * k_st + c);"),
    "merge_adjoint_drops_lse_term": ("dL_parts[p][r] = w * (dot + (gL ? gL[r] : 0.0));",
                                     "dL_parts[p][r] = w * dot;"),
    "sink_adjoint_sign": ("da[h] += -w * (1.0 - w) * dot;", "da[h] += w * (1.0 - w) * dot;"),
    "sink_weight_inverted": ("double w = (l == -INFINITY) ? 0.0 : exp(l - lt);\n            double* o",
                             "double w = (l == -INFINITY) ? 0.0 : exp(lt - l);\n            double* o"),
    "sink_mass_dropped": ("m + log(exp(l - m) + exp(a[h] - m));\n            double w = (l == -INFINITY) ? 0.0 : exp(l - lt);\n            double* o",
                          "m + log(exp(l - m));\n            double w = (l == -INFINITY) ? 0.0 : exp(l - lt);\n            double* o"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTANTS[name]
    text = open(SRC).read()
    # a rule written in several places (forward and backward) is mutated everywhere
    assert text.count(before) >= 1, "mutation site not found: %s" % name
    mutated = tmp_path / "mutant.c"
    mutated.write_text(text.replace(before, after))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99",
                           str(mutated), "-o", str(lib), "-lm"])
    env = dict(os.environ, CPATTN_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
