"""Planted mistakes in the oracle must fail its pins.

Each case copies the oracle's C sources, plants one plausible mistake (a dropped term, a wrong sign,
a wrong index or a transposed operand), builds the copy with the oracle's own compiler flags and
runs the pin tests against it in a subprocess (ATTNRES_ORACLE_LIB points the oracle module at the
copy). A pin suite that still passes would not have caught that mistake. The committed oracle is
never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
SINGLE, MULTI = "attnres_oracle.c", "attnres_oracle_multi.c"

# (name, file, original text, planted text, pin file)
MUTATIONS = [
    ("sum instead of mean in the key RMS", SINGLE,
     "w->r[s] = sqrt(sumsq / R + P->eps);", "w->r[s] = sqrt(sumsq + P->eps);", "single"),
    ("eps outside the square root", SINGLE,
     "w->r[s] = sqrt(sumsq / R + P->eps);", "w->r[s] = sqrt(sumsq / R) + P->eps;", "single"),
    ("key slice taken from the front", SINGLE,
     "const int off = D - R;", "const int off = 0;", "single"),
    ("score without the scale", SINGLE,
     "w->score[s] = P->scale * dot;", "w->score[s] = dot;", "single"),
    ("log-sum-exp without the maximum", SINGLE,
     "const double lse = m + log(l);", "const double lse = log(l);", "single"),
    ("mixture weights of the reversed source order", SINGLE,
     "acc += w->p[s] * value(P, s, n, i);", "acc += w->p[S - 1 - s] * value(P, s, n, i);",
     "single"),
    ("wrong sign of the key-RMS derivative", SINGLE,
     "const double dtj = dkn[j] / r - t[j] * dknt / (R * r * r * r);",
     "const double dtj = dkn[j] / r + t[j] * dknt / (R * r * r * r);", "single"),
    ("softmax gradient without the mean term", SINGLE,
     "w->dscore[s] = w->p[s] * (w->dp[s] - bar);", "w->dscore[s] = w->p[s] * w->dp[s];",
     "single"),
    ("dvalues without the routing weight", SINGLE,
     "= w->p[s] * w->dout_o[i];", "= w->dout_o[i];", "single"),
    ("dq without the scale", SINGLE,
     "w->dq[j] += P->scale * w->dscore[s] * k[j];", "w->dq[j] += w->dscore[s] * k[j];", "single"),
    ("dw from the weighted key instead of the normalised one", SINGLE,
     "if (P->norm_w) w->dw[j] += dk[j] * kn[j];", "if (P->norm_w) w->dw[j] += dk[j] * k[j];",
     "single"),
    ("output-norm backward without its projection term", SINGLE,
     "w->dout_o[i] = rho_o * w->dyhat[i] - rho_o * rho_o * rho_o * go * w->o[i] / D;",
     "w->dout_o[i] = rho_o * w->dyhat[i];", "single"),
    ("dow from the mixture instead of the normalised output", SINGLE,
     "if (P->out_norm && P->out_w) w->dow[i] += g * w->yhat[i];",
     "if (P->out_norm && P->out_w) w->dow[i] += g * w->o[i];", "single"),
    ("multi: dvalues of the last query only", MULTI,
     "for (int i = 0; i < D; ++i) dv[((size_t)s * T + row) * D + i] += p[s] * w->dyv[i];",
     "for (int i = 0; i < D; ++i) dv[((size_t)s * T + row) * D + i] = p[s] * w->dyv[i];", "multi"),
    ("multi: every query's gradient into dq row 0", MULTI,
     "w->dq[(size_t)m * R + j] += P->scale * dscore * k[j];",
     "w->dq[j] += P->scale * dscore * k[j];", "multi"),
    ("multi: dY read token-major (transposed)", MULTI,
     "mload(P->dout, dt, ((int64_t)m * P->N + n) * D + i)",
     "mload(P->dout, dt, ((int64_t)n * P->M + m) * D + i)", "multi"),
    ("multi: key gradient of the last query only", MULTI,
     "dk[j] += P->scale * dscore * mload(P->queries, dt, (int64_t)m * R + j);",
     "dk[j] = P->scale * dscore * mload(P->queries, dt, (int64_t)m * R + j);", "multi"),
    ("selected: bank gradient into slot 0's row", MULTI,
     "double* pe = part + ((size_t)me * P->E + P->ids[n * K + k]) * R;",
     "double* pe = part + ((size_t)me * P->E + P->ids[n * K]) * R;", "multi"),
]

PINS = {"single": "tests/test_oracle_pins.py", "multi": "tests/test_oracle_multi_pins.py"}


@pytest.mark.parametrize("name,fname,old,new,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, name, fname, old, new, pins):
    for f in (SINGLE, MULTI, "attnres_oracle.h"):
        shutil.copy(os.path.join(ORACLE, f), tmp_path / f)
    src = (tmp_path / fname).read_text()
    assert src.count(old) == 1, f"mutation site of '{name}' not found exactly once"
    (tmp_path / fname).write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
                    "-ffp-contract=off", str(tmp_path / SINGLE), str(tmp_path / MULTI),
                    "-o", lib, "-lm"], check=True)
    env = dict(os.environ, ATTNRES_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    # -x: the first failing pin is enough (a full run fails 4 to 18 pins per planted mistake)
    r = subprocess.run([sys.executable, "-m", "pytest", PINS[pins], "-x", "-q", "-p",
                        "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    failed = [l.split()[1] for l in r.stdout.splitlines() if l.startswith("FAILED")]
    print(f"[mutation] {name}: caught by {failed[:1]}", flush=True)
    assert r.returncode == 1 and failed, (
        f"the pins in {PINS[pins]} did not catch '{name}' (exit {r.returncode}):\n"
        f"{r.stdout[-2000:]}\n{r.stderr[-2000:]}")
