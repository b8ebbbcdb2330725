"""Plant plausible mistakes in copies of the oracle and require the pins to see them.

Every mutant is a textual edit of ``oracle/oracle.c`` (a dropped term, a wrong
sign, a wrong index or ordering, a transposed operand).  Each mutant is
compiled into a temporary library and all pin checks run against it in a child
process; at least one check must fail (or the child must crash).
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "phi_missing_plus_one": [("return x > 0.0 ? x + 1.0 : exp(x);", "return x > 0.0 ? x : exp(x);")],
    "la_normalizer_dropped": [("ot[i] = num / den;", "ot[i] = num;")],
    "la_normalizer_not_accumulated": [("z[c] = gam * z[c] + fk[c];", "z[c] = fk[c];")],
    "la_read_before_update": [
        ("for (int i = 0; i < dv; ++i) S[(size_t)c * dv + i] = gam * S[(size_t)c * dv + i] + fk[c] * vt[i];\n                z[c]",
         "for (int i = 0; i < dv; ++i) S[(size_t)c * dv + i] += 0.0;\n                z[c]"),
        ("ot[i] = num / den;", "ot[i] = num / den;\n                for (int c = 0; c < dk; ++c) S[(size_t)c * dv + i] = gam * S[(size_t)c * dv + i] + fk[c] * vt[i];"),
    ],
    "gla_gate_on_value_index": [("gt[c] * S[(size_t)c * dv + i]", "gt[i % dk] * S[(size_t)c * dv + i]")],
    "gla_gate_also_decays_new_write": [
        ("S[(size_t)c * dv + i] = gt[c] * S[(size_t)c * dv + i] + fk[c] * vt[i];",
         "S[(size_t)c * dv + i] = gt[c] * (S[(size_t)c * dv + i] + fk[c] * vt[i]);")],
    "gdr_predict_from_undecayed_state": [
        ("for (size_t e = 0; e < (size_t)dv * dk; ++e) S[e] *= a;", ""),
        ("S[(size_t)i * dk + c] += e * kt[c];", "S[(size_t)i * dk + c] = a * S[(size_t)i * dk + c] + e * kt[c];"),
    ],
    "gdr_error_sign": [("double e = b * (vt[i] - pred[i]);", "double e = b * (vt[i] + pred[i]);")],
    "gdr_beta_dropped": [("double e = b * (vt[i] - pred[i]);", "double e = (vt[i] - pred[i]);")],
    "gdr_gate_index_shift": [("const double a = gate[t];", "const double a = gate[t > 0 ? t - 1 : 0];")],
    "gdr_read_transposed": [("o += S[(size_t)i * dk + c] * qt[c];",
                             "o += S[(size_t)(c % dv) * dk + (i % dk)] * qt[c];")],
    "state_written_transposed": [(": S[(size_t)c * dv + i];", ": S[(size_t)(i % dk) * dv + (c % dv)];")],
    # fixed per-head decay: the page's own pitfall, decaying only one accumulator
    "la_decay_state_only": [("z[c] = gam * z[c] + fk[c];", "z[c] = z[c] + fk[c];")],
    "la_decay_normalizer_only": [
        ("for (int i = 0; i < dv; ++i) S[(size_t)c * dv + i] = gam * S[(size_t)c * dv + i] + fk[c] * vt[i];\n                z[c]",
         "for (int i = 0; i < dv; ++i) S[(size_t)c * dv + i] = S[(size_t)c * dv + i] + fk[c] * vt[i];\n                z[c]")],
    "decay_indexed_by_flat_head": [("return gate + (h % H);", "return gate + (h % (H > 1 ? H : 1) == h ? h : h % H) + (h >= H);")],
    "retention_decays_new_write": [
        ("S[(size_t)c * dv + i] = gam * S[(size_t)c * dv + i] + fk[c] * vt[i];\n            /* y_t",
         "S[(size_t)c * dv + i] = gam * (S[(size_t)c * dv + i] + fk[c] * vt[i]);\n            /* y_t")],
    "kda_decay_on_value_rows": [("for (int c = 0; c < dk; ++c) S[(size_t)i * dk + c] *= alpha[c];",
                                 "for (int c = 0; c < dk; ++c) S[(size_t)i * dk + c] *= alpha[i % dk];")],
    "kda_predict_from_undecayed_state": [
        ("for (int c = 0; c < dk; ++c) S[(size_t)i * dk + c] *= alpha[c];", ""),
        ("for (int c = 0; c < dk; ++c) S[(size_t)i * dk + c] += err * kt[c];",
         "for (int c = 0; c < dk; ++c) S[(size_t)i * dk + c] = alpha[c] * S[(size_t)i * dk + c] + err * kt[c];")],
    "kda_beta_dropped": [("const double err = bw * (vt[i] - pred[i]);", "const double err = (vt[i] - pred[i]);")],
    # gradients
    "bwd_normalizer_cotangent_sign": [("dden = -dot_o / den;", "dden = dot_o / den;")],
    "bwd_normalizer_cotangent_dropped": [("s += dden * zt[c];", "s += 0.0 * zt[c];")],
    "bwd_phi_prime_dropped": [("return x > 0.0 ? 1.0 : exp(x);", "return 1.0;")],
    "bwd_state_cotangent_not_decayed": [("for (size_t e = 0; e < sz; ++e) dS[e] *= gam;", "")],
    "bwd_decay_grad_misses_normalizer": [("for (int c = 0; c < dk; ++c) dg += dz[c] * zp[c];", "")],
    "bwd_decay_grad_uses_new_state": [("for (size_t e = 0; e < sz; ++e) dg += dS[e] * Sp[e];",
                                       "for (size_t e = 0; e < sz; ++e) dg += dS[e] * St[e];")],
    "bwd_key_grad_misses_normalizer": [("        s += dz[c];\n", "")],
    "bwd_value_grad_uses_query": [("for (int c = 0; c < dk; ++c) s += dS[(size_t)c * dv + i] * fk[c];",
                                   "for (int c = 0; c < dk; ++c) s += dS[(size_t)c * dv + i] * fq[c];")],
    "initial_state_ignored_for_gla": [("else                              S[(size_t)c * dv + i] = s;",
                                       "else                              S[(size_t)c * dv + i] = (variant == 1) ? 0.0 : s;")],
}

CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
from oracle_pin_checks import ALL_CHECKS
orc = oracle.load({lib!r})
failed = []
for chk in ALL_CHECKS:
    try:
        chk(orc)
    except Exception as e:
        failed.append(chk.__name__)
print("FAILED:" + ",".join(failed))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, "mutation target not found exactly once: %r" % old
        src = src.replace(old, new)
    msrc = tmp_path / "oracle_mutant.c"
    msrc.write_text(src)
    lib = oracle.build(force=True, src=str(msrc), out=str(tmp_path / "libmutant.so"))
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    if res.returncode != 0:
        return  # a crash is a detection too
    line = [l for l in res.stdout.splitlines() if l.startswith("FAILED:")][-1]
    failed = [f for f in line[len("FAILED:"):].split(",") if f]
    assert failed, "mutant %s passed every pin" % name
