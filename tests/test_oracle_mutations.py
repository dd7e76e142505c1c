"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (a dropped or
repeated term, a flipped sign, a wrong index or stride, a changed rounding
order or precision), builds the copy with gcc, and runs the oracle pin tests
against it in a separate process: at least one pin must fail.  A control run
of the unchanged copy through the same harness must pass, so a broken harness
cannot make every mistake look caught.  Everything here runs on the CPU; the
GPU path is not involved.
"""
import os
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

import oracle

ROOT = Path(__file__).resolve().parents[1]
PIN_TESTS = [ROOT / "tests" / "test_oracle_diffusion.py", ROOT / "tests" / "test_oracle_pack_flux.py"]

# (name, text in oracle.c, replacement, which occurrence: 0 = first)
MUTATIONS = [
    # five-point update, FP64 (Qiita Part 3, section 3)
    ("f64 south read from the north", "t = t + src[p - ld];                /* + S  (j - 1)   */",
     "t = t + src[p + ld];", 0),
    ("f64 plus four c", "t = t - four * c;                   /* - 4 C          */", "t = t + four * c;", 0),
    ("f64 west dropped for east", "double t = src[p - 1] + src[p + 1]; /* W + E          */",
     "double t = src[p + 1] + src[p + 1];", 0),
    ("f64 (W+E)+(S+N) order", "t = t + src[p - ld];                /* + S  (j - 1)   */\n"
     "                t = t + src[p + ld];                /* + N  (j + 1)   */",
     "t = t + (src[p - ld] + src[p + ld]);", 0),
    ("f64 centre term dropped", "dst[p] = c + a * t;", "dst[p] = a * t;", 0),
    ("f64 fused multiply-add", "dst[p] = c + a * t;", "dst[p] = __builtin_fma(a, t, c);", 0),
    # the same update in FP32
    ("f32 west dropped for east", "float t = src[p - 1] + src[p + 1];", "float t = src[p + 1] + src[p + 1];", 0),
    ("f32 sum carried in double", "float t = src[p - 1] + src[p + 1];", "double t = src[p - 1] + src[p + 1];", 0),
    # directional pack and its inverse (MFC pull request 2087)
    ("y pack in x order", "o = k + ny * (j + nx * (l + nz * (int64_t)var));",
     "o = j + nx * (k + ny * (l + nz * (int64_t)var));", 0),
    ("z pack with j and k swapped", "o = l + nz * (k + ny * (j + nx * (int64_t)var));",
     "o = l + nz * (j + nx * (k + ny * (int64_t)var));", 0),
    ("y unpack in x order", "o = k + ny * (j + nx * (l + nz * (int64_t)var));",
     "o = j + nx * (k + ny * (l + nz * (int64_t)var));", 1),
    # conservative flux difference
    ("x high face with the cell stride", "fx[var][(j + 1) + (nx + 1) * (k + ny * l)]) *",
     "fx[var][(j + 1) + nx * (k + ny * l)]) *", 0),
    ("y spacing indexed by j", "const double iy = 1.0 / dy[k];", "const double iy = 1.0 / dy[j % ny];", 0),
    ("z high face is the low face", "fz[var][j + nx * (k + ny * (l + 1))]) *", "fz[var][j + nx * (k + ny * l)]) *", 0),
    ("y term subtracted", "r = r + (fy[var]", "r = r - (fy[var]", 0),
    ("x term divided instead of multiplied by the reciprocal", "const double ix = 1.0 / dx[j];",
     "const double ix = 1.0 / dx[j]; const double dxj = dx[j];", 0),
    # SSPRK stage
    ("stage adds to q0 instead of q", "t = q[var][c] + t;", "t = q0[var][c] + t;", 0),
    ("stage subtracts the two parts", "qout[var][c] = s + t;", "qout[var][c] = s - t;", 0),
    ("stage with b distributed", "double t = dt * rhs[c + n * var];\n            t = q[var][c] + t;\n            t = b * t;",
     "double t = b * (dt * rhs[c + n * var]);\n            t = b * q[var][c] + t;", 0),
]

# The division form needs the multiply rewritten too.
FOLLOW_UPS = {
    "x term divided instead of multiplied by the reciprocal": [
        ("fx[var][(j + 1) + (nx + 1) * (k + ny * l)]) *\n                               ix;",
         "fx[var][(j + 1) + (nx + 1) * (k + ny * l)]) /\n                               dxj;"),
    ],
}


def _replace_nth(text, old, new, nth):
    at = -1
    for _ in range(nth + 1):
        at = text.find(old, at + 1)
        assert at >= 0, f"mutation anchor not found: {old!r}"
    return text[:at] + new + text[at + len(old):]


def _run_pins(tmp_path, source):
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    shutil.copy(ROOT / "oracle" / "__init__.py", pkg / "__init__.py")
    (pkg / "oracle.c").write_text(source)
    # Built here, with the oracle's own flags, so that a mistake that does not
    # compile cannot pass for one the pins caught.
    subprocess.run(["gcc", *oracle.GCC_FLAGS, str(pkg / "oracle.c"), "-o", str(pkg / "liboracle.so")],
                   check=True, capture_output=True, timeout=120)
    env = dict(os.environ)
    # The copy comes first: the working directory (the temporary one) heads
    # sys.path under `python -m`, and the repository supplies the inputs module.
    env["PYTHONPATH"] = os.pathsep.join([str(tmp_path), str(ROOT)])
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           "-c", str(ROOT / "pytest.ini"), "--rootdir", str(ROOT), *map(str, PIN_TESTS)]
    return subprocess.run(cmd, cwd=tmp_path, env=env, capture_output=True, text=True, timeout=600)


def _which_oracle(tmp_path):
    env = dict(os.environ)
    env["PYTHONPATH"] = os.pathsep.join([str(tmp_path), str(ROOT)])
    out = subprocess.run([sys.executable, "-c", "import oracle; print(oracle.__file__)"], cwd=tmp_path,
                         env=env, capture_output=True, text=True, timeout=120)
    return out.stdout.strip()


def test_control_copy_passes_and_is_the_one_loaded(tmp_path):
    source = (ROOT / "oracle" / "oracle.c").read_text()
    res = _run_pins(tmp_path, source)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
    assert _which_oracle(tmp_path) == str(tmp_path / "oracle" / "__init__.py")


@pytest.mark.parametrize("name,old,new,nth", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, name, old, new, nth):
    source = (ROOT / "oracle" / "oracle.c").read_text()
    mutated = _replace_nth(source, old, new, nth)
    for a, b in FOLLOW_UPS.get(name, []):
        mutated = _replace_nth(mutated, a, b, 0)
    assert mutated != source
    res = _run_pins(tmp_path, mutated)
    assert res.returncode == 1, f"no pin caught: {name} (exit {res.returncode})\n" + res.stdout[-1500:]
    assert " failed" in res.stdout, res.stdout[-1500:]
