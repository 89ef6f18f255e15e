"""The oracle's pins catch plausible mistakes (CPU only).

Each case copies the oracle package to a temporary directory, plants one mistake in the copy
(the C forward oracle, or the numpy backward and packed-batch oracles), and runs the pin tests
that cover it (tests/test_oracle.py, test_oracle_bwd.py, test_oracle_varlen.py) against the
copy in a child process: they must fail. The unmutated copy must pass the same tests, so a
failure is the mistake's doing and not the copy's.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")

C, PY = "attn_oracle.c", "__init__.py"
FWD, BWD, VARLEN = "test_oracle.py", "test_oracle_bwd.py", "test_oracle_varlen.py"

# (name, file, original text, mutated text, pin tests to run)
MUTATIONS = [
    ("fwd: dropped first head-dim term of q.k", C,
     "for (int64_t c = 0; c < d; ++c)\n            dot += qi[c] * kh[j * d + c];",
     "for (int64_t c = 1; c < d; ++c)\n            dot += qi[c] * kh[j * d + c];", [FWD]),
    ("fwd: wrong sign of the scale", C, "s[j] = J->scale * dot;", "s[j] = -J->scale * dot;", [FWD]),
    ("fwd: transposed K operand", C, "dot += qi[c] * kh[j * d + c];", "dot += qi[c] * kh[c * Nk + j];", [FWD]),
    ("fwd: causal mask drops the diagonal", C, "int valid = !J->causal || j <= i;",
     "int valid = !J->causal || j < i;", [FWD]),
    ("fwd: causal mask shows one key too many", C, "int valid = !J->causal || j <= i;",
     "int valid = !J->causal || j <= i + 1;", [FWD]),
    ("fwd: K in place of V", C, "acc += s[j] * vh[j * d + c];", "acc += s[j] * kh[j * d + c];", [FWD]),
    ("fwd: missing division by the row sum", C, "o_row[c] = acc / l;", "o_row[c] = acc;", [FWD]),
    ("fwd: L without the row max", C, "*lse_out = m + log(l);", "*lse_out = log(l);", [FWD]),
    ("fwd: L in base 2", C, "*lse_out = m + log(l);", "*lse_out = m + log2(l);", [FWD]),
    ("bwd: dropped D term of dS", PY, "ds = p * (dp - D)", "ds = p * dp", [BWD]),
    ("bwd: row term from the stored output without dO", PY,
     "D = (do[b, h] * o[b, h]).sum(axis=1, keepdims=True)", "D = o[b, h].sum(axis=1, keepdims=True)", [BWD]),
    ("bwd: missing scale in dQ", PY, "dq[b, h] = scale * (ds @ k[b, h])", "dq[b, h] = ds @ k[b, h]", [BWD]),
    ("bwd: K in place of V in dP", PY, "dp = do[b, h] @ v[b, h].T", "dp = do[b, h] @ k[b, h].T", [BWD]),
    ("bwd: causal mask one key too wide", PY,
     "visible = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None]",
     "visible = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + 1", [BWD]),
    ("bwd: scaled dV", PY, "dv[b, h] = p.T @ do[b, h]", "dv[b, h] = scale * (p.T @ do[b, h])", [BWD]),
    ("varlen: values of the wrong sequence", PY, "v[None, :, ks:ke]", "v[None, :, qs:qs + (ke - ks)]", [VARLEN]),
    ("varlen: keyless rows not left empty", PY, "if qe == qs or ke == ks:", "if qe == qs:", [VARLEN]),
]


def _mutant(tmp_path, fname=None, old=None, new=None):
    dst = tmp_path / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), dst,
                    ignore=shutil.ignore_patterns("*.so", "*.so.tmp*", "__pycache__"))
    if fname is not None:
        path = dst / fname
        text = path.read_text()
        assert text.count(old) == 1, f"{fname}: the original text must occur exactly once: {old!r}"
        path.write_text(text.replace(old, new))
    return str(tmp_path)


def _run_pins(mutant_dir, files):
    env = dict(os.environ, ORACLE_MUTANT_DIR=mutant_dir, PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join(TESTS, f) for f in files]]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_unmutated_copy_passes_the_pins(tmp_path):
    r = _run_pins(_mutant(tmp_path), [FWD, BWD, VARLEN])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    # the child imported the copy, not the repository's package
    assert os.path.exists(tmp_path / "oracle" / "libattn_oracle.so")


@pytest.mark.parametrize("name,fname,old,new,files", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, name, fname, old, new, files):
    r = _run_pins(_mutant(tmp_path, fname, old, new), files)
    # exit status 1: tests ran and at least one failed (2-5 would be a usage or collection error)
    assert r.returncode == 1, f"{name}: pins did not fail (rc {r.returncode})\n{r.stdout[-2000:]}"
