"""The oracle's pins must catch plausible mistakes.

Each case plants one slip in a copy of oracle/mbref.c (a flipped tie-break,
the other move-size reading, a lost term, a transposed index, ...), builds it
into a temporary library and runs the pin suite against it in a subprocess;
the suite has to fail. All on the CPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mbref.c")

# (name, original text, mutated text)
MUTANTS = [
    ("busiest rank tie -> highest index",
     "if (load[r] - tau[r] > load[rs] - tau[rs]) rs = r;",
     "if (load[r] - tau[r] >= load[rs] - tau[rs]) rs = r;"),
    ("heaviest expert tie -> highest id",
     "if (best < 0 || qh[e] > qh[best]) best = e;", "if (best < 0 || qh[e] >= qh[best]) best = e;"),
    ("destination tie -> highest index",
     "if (dst < 0 || tau[r] - load[r] > tau[dst] - load[dst]) dst = r;",
     "if (dst < 0 || tau[r] - load[r] >= tau[dst] - load[dst]) dst = r;"),
    ("destination -> most loaded open rank",
     "if (dst < 0 || tau[r] - load[r] > tau[dst] - load[dst]) dst = r;",
     "if (dst < 0 || tau[r] - load[r] < tau[dst] - load[dst]) dst = r;"),
    ("move size capped at the busiest rank's excess",
     "int64_t m = tau[dst] - load[dst];",
     "int64_t m = tau[dst] - load[dst];\n      if (load[rs] - tau[rs] < m) m = load[rs] - tau[rs];"),
    ("water level one below the ceiling",
     "tau[r] = (N * K * sr + sum_s - 1) / sum_s;", "tau[r] = (N * K * sr + sum_s - 1) / sum_s - 1;"),
    ("busiest rank by load, not by excess over its target",
     "if (load[r] - tau[r] > load[rs] - tau[rs]) rs = r;", "if (load[r] > load[rs]) rs = r;"),
    ("destination by least load, not by deficit under its target",
     "if (dst < 0 || tau[r] - load[r] > tau[dst] - load[dst]) dst = r;",
     "if (dst < 0 || load[r] < load[dst]) dst = r;"),
    ("weighted targets rounded down",
     "tau[r] = (N * K * sr + sum_s - 1) / sum_s;", "tau[r] = (N * K * sr) / sum_s;"),
    ("speeds ignored",
     "const int64_t sr = speed ? speed[r] : 1;", "const int64_t sr = 1;"),
    ("highest free slot",
     "while (o->rep_expert[dst * R + j] >= 0) ++j;", "j = R - 1;\n      while (o->rep_expert[dst * R + j] >= 0) --j;"),
    ("no local preference (pass 1 off)",
     "if (is_host[e * P + s] && used[e * P + s] < Q[e * P + s]) {", "if (0) {"),
    ("surplus to the highest-index host",
     "int64_t h = 0;\n      while (h < P && !(is_host[e * P + h] && used[e * P + h] < Q[e * P + h])) ++h;",
     "int64_t h = P - 1;\n      while (h >= 0 && !(is_host[e * P + h] && used[e * P + h] < Q[e * P + h])) --h;\n      if (h < 0) h = P;"),
    ("replica slots numbered before home slots",
     "slot_of[h * E + e] = e - h * Eh;", "slot_of[h * E + e] = R + e - h * Eh;"),
    ("token source is t % P",
     "const int64_t s = t / S;\n    for (int64_t k = 0; k < K; ++k) o->counts[s * E + ids[t * K + k]] += 1;",
     "const int64_t s = t % P;\n    for (int64_t k = 0; k < K; ++k) o->counts[s * E + ids[t * K + k]] += 1;"),
    ("combine drops the last expert",
     "for (int64_t k = 0; k < K; ++k) {\n        const double v = out_elem", "for (int64_t k = 0; k < K - 1; ++k) {\n        const double v = out_elem"),
    ("combine ignores the weights",
     "const double term = (double)w[t * K + k] * v;", "const double term = v / (double)K;"),
    ("dispatch copies the next token",
     "memcpy((char*)buf_win + (p - row0) * rb, (const char*)x + t * rb, (size_t)rb);",
     "memcpy((char*)buf_win + (p - row0) * rb, (const char*)x + ((t + 1) % N) * rb, (size_t)rb);"),
    ("drift reference not accumulated",
     "for (int64_t e = 0; e < E; ++e) st->wsum[e] += c[e];", "for (int64_t e = 0; e < 0; ++e) st->wsum[e] += c[e];"),
    ("drift reference not restarted at a replan",
     "for (int64_t e = 0; e < E; ++e) st->wsum[e] = c[e];", "for (int64_t e = 0; e < E; ++e) st->wsum[e] += c[e];"),
    ("drift threshold inclusive",
     "if (st->last_d > (double)prm->delta_num", "if (st->last_d >= (double)prm->delta_num"),
    ("drift check on every call",
     "if (!replan && --st->countdown == 0) {", "if (!replan && (--st->countdown, 1)) {"),
    ("drift distance without the norms' square roots",
     "(sqrt((double)n1) * sqrt((double)n2))", "((double)n1 + (double)n2)"),
    ("kept replica takes pairs whatever its home's load",
     "if (load[h] > tau[h] && load[dst] < tau[dst]) {", "if (load[dst] < tau[dst]) {"),
    ("repair moves quota one way only",
     "        *qb += t;\n        *qa -= t;\n        left_ba -= t;", "        left_ba -= t;"),
    ("repair cancels the larger flow",
     "int64_t left_ab = fab < fba ? fab : fba, left_ba = left_ab;",
     "int64_t left_ab = fab > fba ? fab : fba, left_ba = left_ab;"),
    ("circle method without rotation",
     "*a = pa == 0 ? 0 : 1 + (pa - 1 + round) % (n - 1);", "*a = pa == 0 ? 0 : 1 + (pa - 1) % (n - 1);"),
    ("repair misses replicas of a's home experts on b",
     "if (e >= 0 && e / Eh == a) common[nc++] = e;", "if (0) common[nc++] = e;"),
    ("repair skips pairs with the last rank",
     "if (a >= P || b >= P) continue; /* bye */", "if (a >= P - 1 || b >= P - 1) continue;"),
    ("fp8 combine scale of the wrong block",
     "(double)y_scale[p * (H / 128) + i / 128];", "(double)y_scale[p * (H / 128) + i / 256];"),
    ("fp8 decode without the subnormal range",
     "    v = ldexp((double)m, -9);", "    v = ldexp(1.0 + m / 8.0, -7);"),
    ("load guard ignores the region size",
     "    if (load > dm->cap) return 0;\n", ""),
    ("load guard tolerance exclusive",
     "if (prm->tol_den > 0 && load * prm->tol_den > tau", "if (prm->tol_den > 0 && load * prm->tol_den >= tau"),
    ("load guard against the largest target",
     "const int64_t tau = (NK * (speed ? speed[r] : 1) + sum_s - 1) / sum_s;",
     "const int64_t tau = (NK * (speed ? speed[P - 1] : 1) + sum_s - 1) / sum_s;"),
    ("load guard flags the call but keeps the replay",
     "      replan = 1;\n      guarded = 1;", "      guarded = 1;"),
    ("duplicate ids not flagged",
     "if (ids[t * K + k2] == e) flags |= MBREF_ST_DUP_ID;", "if (0) flags |= MBREF_ST_DUP_ID;"),
]

FAST_PINS = "not prefill and not decode_drift_sequence and not dsv3 and not milp"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mutated = src.replace(old, new, 1)
    c = tmp_path / "mbref.c"
    c.write_text(mutated)
    (tmp_path / "mbref.h").write_text(open(os.path.join(ROOT, "oracle", "mbref.h")).read())
    lib = tmp_path / "libmbref_mutant.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-ffp-contract=off", "-shared", "-fPIC", "-o", str(lib),
                    str(c), "-lm"], check=True, capture_output=True)
    env = dict(os.environ, MBREF_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", "-k", FAST_PINS,
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch: {name}\n{r.stdout[-2000:]}"
