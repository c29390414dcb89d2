"""Plant plausible mistakes in a copy of the oracle and check that the pins catch each one.

Every mutant is a textual edit of oracle/lola_oracle.c compiled into a temporary
library (the real oracle source is never touched).  A mutant that passes every
pin would mean the pins leave that part of the oracle unchecked.
"""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins as P

MUTANTS = {
    "drop_pending_term": [("if (Rpos[i] > t - w) continue;", "if (1) continue;")],
    "window_one_too_wide": [("Rpos[i] < t - w + 1) continue;", "Rpos[i] < t - w) continue;")],
    "sre_wrong_sign": [("double diff = r - v[j];", "double diff = r + v[j];")],
    "sre_wrong_state_column": [("n += phik[i] * H[(size_t)i * D + j];",
                                "n += phik[i] * H[(size_t)i * D + (D - 1 - j)];")],
    "keep_lowest_scores": [("if (a->e > b->e) return -1;", "if (a->e > b->e) return 1;"),
                           ("if (a->e < b->e) return 1;", "if (a->e < b->e) return -1;")],
    "tie_prefers_newer": [("if (a->pos < b->pos) return -1;", "if (a->pos < b->pos) return 1;"),
                          ("if (a->pos > b->pos) return 1;", "if (a->pos > b->pos) return -1;")],
    "phi_second_half_not_negated": [("out[Fh + i] = exp(-z[i] + zmin);", "out[Fh + i] = exp(z[i] - zmax);")],
    "fold_skips_normaliser": [("c->s[i] += ph[i];", "c->s[i] += 0.0 * ph[i];")],
    "no_softmax_scale": [("lg[nl] = tau * dot;", "lg[nl] = dot;")],
    "leaving_set_one_short": [("Rpos[nE] <= e - 1 - w) ++nE;", "Rpos[nE] < e - 1 - w) ++nE;")],
    "readout_drops_state": [("acc += phq[i] * c->H[(size_t)i * D + j];", "acc += 0.0 * c->H[(size_t)i * D + j];")],
    "linear_not_rescaled": [("double sc = exp(-m);", "double sc = 1.0;")],
    "window_keeps_one_less": [("if (Rpos[i] < e - w) continue;", "if (Rpos[i] < e - w + 1) continue;")],
    "fold_transposed_value": [("c->H[(size_t)i * D + j] += ph[i] * Uv[u][j];",
                               "c->H[(size_t)i * D + j] += ph[i] * Uv[u][D - 1 - j];")],
    # teacher forcing (a kept set adopted from outside)
    "forced_set_of_wrong_head": [("jb->forced + (((size_t)b * Hkv + g) * jb->NI + ci)",
                                  "jb->forced + (((size_t)b * Hkv + 0) * jb->NI + ci)")],
    "forced_set_of_first_interval": [("jb->forced + (((size_t)b * Hkv + g) * jb->NI + ci)",
                                      "jb->forced + (((size_t)b * Hkv + g) * jb->NI + 0)")],
    # scoring and cache policies other than the SRE
    "stale_scores_refreshed": [("for (int u = 0; u < c->cn; ++u) cand[u].e = c->cscore[u];",
                                "for (int u = 0; u < c->cn; ++u) cand[u].e += 0.0 * c->cscore[u];")],
    "fifo_keeps_oldest": [("for (int u = 0; u < nU; ++u) cand[u].e = (double)Upos[u];",
                           "for (int u = 0; u < nU; ++u) cand[u].e = -(double)Upos[u];")],
    "attn_weights_not_normalised": [("const double p = exp(lgt[u] - mx) / zs;",
                                     "const double p = exp(lgt[u] - mx) / (zs > 0.0 ? 1.0 : zs);")],
    "scorers_use_first_query": [("const int64_t tl = e - 1;", "const int64_t tl = a;")],
    "kerr_signed_difference": [("fabs(p - kap[u] / ks)", "(p - kap[u] / ks)")],
    "forced_kept_pair_also_folded": [("        if (keep[u]) continue;\n        const double* ph = Uphi",
                                      "        if (keep[u] && !(jb->forced && u == 0)) continue;\n"
                                      "        const double* ph = Uphi")],
}


def _mutant_lib(tmp_path, name, edits):
    with open(oracle.SRC) as f:
        src = f.read()
    for old, new in edits:
        assert old in src, f"mutant {name}: snippet not found: {old}"
        src = src.replace(old, new)
    path = os.path.join(tmp_path, f"mut_{name}.c")
    with open(path, "w") as f:
        f.write(src)
    so = os.path.join(tmp_path, f"libmut_{name}.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", so, path, "-lm", "-lpthread"],
                   check=True)
    return oracle.load(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    lib = _mutant_lib(str(tmp_path), name, MUTANTS[name])
    caught = []
    for check in P.ALL_CHECKS:
        try:
            check(lib)
        except (AssertionError, ValueError, RuntimeError, FloatingPointError):
            caught.append(check.__name__)
    assert caught, f"no pin detects the planted mistake {name}"
