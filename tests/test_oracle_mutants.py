"""The oracle's pins must catch plausible mistakes in the oracle.

Each case below plants one mistake in a copy of the oracle's C source (a
dropped term, a wrong index or sign, a transposed operand, a wrong rounding
rule), builds it on the CPU, and runs the oracle pin tests against that build;
the Python-level cases plant one mistake in the composition layer
(oracle/__init__.py: token slicing, operand order, pattern dispatch) and run
the pins with the mutated module source executed over the real one. The pin
suite has to fail for every one of them; a mutant that passes means a part of
the oracle is not pinned.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_codecs.py", "tests/test_oracle_norm.py",
             "tests/test_oracle_quant.py", "tests/test_oracle_qk.py", "tests/test_oracle_sharded.py",
             "tests/test_oracle_static.py", "tests/test_oracle_ag.py", "tests/test_oracle_rs.py"]
PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")

# (name, text in the source, replacement)
MUTANTS = [
    ("drops the last partial",
     "for (int p = 0; p < P; ++p) acc +=", "for (int p = 0; p < P - 1; ++p) acc +="),
    ("forgets the residual",
     "x[j] = acc + (float)orc_bf16_decode(residual[row_off + j]);", "x[j] = acc;"),
    ("sums the partials in fp64",
     "float acc = 0.0f;", "double acc = 0.0;"),
    ("adds the residual first",
     "float acc = 0.0f;\n        for (int p = 0; p < P; ++p) acc += (float)orc_bf16_decode("
     "partials[p][row_off + j]);\n        x[j] = acc + (float)orc_bf16_decode(residual[row_off"
     " + j]);",
     "float acc = (float)orc_bf16_decode(residual[row_off + j]);\n        for (int p = 0; p < P;"
     " ++p) acc += (float)orc_bf16_decode(partials[p][row_off + j]);\n        x[j] = acc;"),
    ("mean over H - 1",
     "double ms = ss / (double)H;", "double ms = ss / (double)(H - 1);"),
    ("eps outside the sqrt",
     "return 1.0 / sqrt(ms + (double)eps);", "return 1.0 / (sqrt(ms) + (double)eps);"),
    ("weight used as 1 + w",
     "y[j] = (double)x[j] * inv * orc_bf16_decode(weight[j]);",
     "y[j] = (double)x[j] * inv * (1.0 + orc_bf16_decode(weight[j]));"),
    ("weight index reversed",
     "y[j] = (double)x[j] * inv * orc_bf16_decode(weight[j]);",
     "y[j] = (double)x[j] * inv * orc_bf16_decode(weight[H - 1 - j]);"),
    ("bf16 truncates instead of rounding",
     "if (rem > 0.5 || (rem == 0.5 && fmod(n, 2.0) != 0.0)) n += 1.0;", ""),
    ("bf16 ties away from zero",
     "(rem == 0.5 && fmod(n, 2.0) != 0.0)", "(rem == 0.5)"),
    ("e4m3 exponent bias 8",
     "v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("e4m3 subnormal scale",
     "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    ("e4m3 ties to odd",
     "if (dhi < dlo || (dhi == dlo && (c & 1))) c += 1;",
     "if (dhi < dlo || (dhi == dlo && !(c & 1))) c += 1;"),
    ("e4m3 does not saturate",
     "if (a > 448.0) a = 448.0;\n    int c = orc_e4m3_floor_code(a);\n    if (c < 126)",
     "int c = orc_e4m3_floor_code(a);\n    if (a > 448.0) return (uint8_t)(sign | 0x7F);\n"
     "    if (c < 126)"),
    ("scale stored as the quantisation multiplier",
     "*scale = (float)(amax / 448.0);", "*scale = (float)(448.0 / amax);"),
    ("quantises against the wrong maximum",
     "double r = 448.0 * y[j] / amax;", "double r = 448.0 * y[j] / (2.0 * amax);"),
    ("block scales transposed",
     "scales + t * n_groups + g", "scales + g * T + t"),
    ("QK ignores tp_world",
     "double inv_q = 1.0 / sqrt(vq / (double)tp_world + (double)eps);",
     "double inv_q = 1.0 / sqrt(vq + (double)eps);"),
    ("QK k statistics read v",
     "double v = orc_bf16_decode(row[q_size + j]);\n            sk += v * v;\n        }\n"
     "        means",
     "double v = orc_bf16_decode(row[q_size + kv_size + j]);\n            sk += v * v;\n"
     "        }\n        means"),
    ("QK mean over the wrong width",
     "vk = sk / (double)kv_size;", "vk = sk / (double)q_size;"),
    ("QK k output uses q's weight",
     "inv_k * orc_bf16_decode(k_weight[j])", "inv_k * orc_bf16_decode(q_weight[j])"),
    ("static scale multiplies instead of dividing",
     "double r = y / s;", "double r = y * s;"),
    ("static codes from bf16(y)",
     "codes[off + j] = orc_e4m3_encode(r);",
     "codes[off + j] = orc_e4m3_encode(orc_bf16_decode(orc_bf16_encode(y)) / s);"),
    ("MLA y segment takes the x eps",
     "double inv_y = 1.0 / sqrt(sy / (double)kv_rank + (double)y_eps);",
     "double inv_y = 1.0 / sqrt(sy / (double)kv_rank + (double)x_eps);"),
    ("MLA y segment reads the rope part",
     "double v = orc_bf16_decode(row[q_rank + j]);\n                sy += v * v;",
     "double v = orc_bf16_decode(row[row_stride - kv_rank + j]);\n                sy += v * v;"),
    ("sharded norm ignores tp_world",
     "double inv = 1.0 / sqrt(var / (double)tp_world + (double)eps);",
     "double inv = 1.0 / sqrt(var + (double)eps);"),
    ("sharded means over H - 1",
     "means[t] = ss / (double)H;", "means[t] = ss / (double)(H - 1);"),
    ("sharded norm eps outside the sqrt",
     "double inv = 1.0 / sqrt(var / (double)tp_world + (double)eps);",
     "double inv = 1.0 / (sqrt(var / (double)tp_world) + (double)eps);"),
]


# (name, text in oracle/__init__.py, replacement)
PY_MUTANTS = [
    ("RS slice starts one row late",
     "np.asarray(p)[token_offset:token_offset + T]",
     "np.asarray(p)[token_offset + 1:token_offset + 1 + T]"),
    ("RS adds add_in before the partials",
     "rows.append(_c(add_in, np.uint16))", "rows.insert(0, _c(add_in, np.uint16))"),
    ("RS adds add_in after the residual",
     "        rows.append(_c(add_in, np.uint16))\n",
     "        residual, rows = _c(add_in, np.uint16), rows + [_c(residual, np.uint16)]\n"),
    ("RS pattern 4 writes no norm",
     "want_norm=pattern == RS_RESIDUAL_RMSNORM_OUT_FP8", "want_norm=False"),
    ("RS static patterns ignore the scale",
     "fused_add_rmsnorm_static(rows, residual, weight, eps, scale_factor,",
     "fused_add_rmsnorm_static(rows, residual, weight, eps, 1.0,"),
]

# Runs the pins with a mutated oracle/__init__.py executed over the imported module.
_PY_DRIVER = """import sys
import oracle
exec(compile(open(sys.argv[1]).read(), oracle.__file__, "exec"), oracle.__dict__)
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", *sys.argv[2:]]))
"""


def _run_py_mutant(case, tmp):
    name, old, new = case
    with open(PY_SRC) as f:
        src = f.read()
    if src.count(old) != 1:
        return name, "pattern not found exactly once"
    path = os.path.join(tmp, f"py{abs(hash(name))}.py")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", _PY_DRIVER, path, *PIN_FILES], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    if r.returncode == 0:
        return name, "SURVIVED: no pin failed"
    if r.returncode != 1:
        return name, f"pytest exited {r.returncode}: " + r.stdout[-400:]
    return name, None


def _run_mutant(case, tmp):
    name, old, new = case
    with open(_build.SRC) as f:
        src = f.read()
    if src.count(old) != 1:
        return name, "pattern not found exactly once"
    path = os.path.join(tmp, f"m{abs(hash(name))}.c")
    lib = path[:-2] + ".so"
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    b = subprocess.run(["gcc", *_build.CFLAGS, path, "-o", lib, "-lm"], capture_output=True,
                       text=True)
    if b.returncode != 0:
        return name, "mutant did not compile: " + b.stderr[-400:]
    env = dict(os.environ, FUSEDNORM_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    if r.returncode == 0:
        return name, "SURVIVED: no pin failed"
    if r.returncode != 1:   # 1 = tests failed; anything else is an error in the harness
        return name, f"pytest exited {r.returncode}: " + r.stdout[-400:]
    return name, None


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda c: _run_mutant(c, tmp), MUTANTS))
            results += list(ex.map(lambda c: _run_py_mutant(c, tmp), PY_MUTANTS))
    bad = [f"{n}: {msg}" for n, msg in results if msg]
    assert not bad, "\n".join(bad)


@pytest.mark.parametrize("case", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutation_pattern_is_present(case):
    with open(_build.SRC) as f:
        assert f.read().count(case[1]) == 1


@pytest.mark.parametrize("case", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_python_mutation_pattern_is_present(case):
    with open(PY_SRC) as f:
        assert f.read().count(case[1]) == 1
