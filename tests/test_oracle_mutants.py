"""Plant plausible mistakes in a copy of the C oracle (CPU only) and check that
the pins catch every one of them.  The oracle source itself is untouched; each
variant is compiled into a temporary directory and exercised in a child
process (a mistaken index may read outside an array)."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gqa_oracle.c")

# (name, text in the oracle source, replacement)
MUTANTS = [
    ("drop_scale", "double sj = scale * dot;", "double sj = dot;"),
    ("head_mapping_mod", "int kv = h / G;", "int kv = h % H_kv;"),
    ("diagonal_excluded", "(int64_t)q_offset + t + 1", "(int64_t)q_offset + t + (t == 0)"),
    ("q_offset_ignored", "(int64_t)q_offset + t + 1", "(int64_t)t + 1"),
    ("lse_without_max", "lse[i] = m + log(l);", "lse[i] = log(l);"),
    ("no_normalisation", "o[i * d + x] = acc[x] / l;", "o[i * d + x] = acc[x];"),
    ("no_normalisation_decode", "o[i * d + x] = run[x] / l;", "o[i * d + x] = run[x];"),
    ("v_reads_k", "const float *vrow = vbase + j * stride;",
     "const float *vrow = kbase + j * stride;"),
    ("exp_sign", "double p = exp(s[j - j0] - m);", "double p = exp(m - s[j - j0]);"),
    ("q_dot_q", "dot += (double)qrow[x] * (double)krow[x];",
     "dot += (double)qrow[x] * (double)qrow[x];"),
    ("key_stride", "const int64_t kstride = (int64_t)H_kv * d;",
     "const int64_t kstride = (int64_t)d;"),
    ("merge_sign", "double sa = (m == -INFINITY) ? 0.0 : exp(m - mm);",
     "double sa = (m == -INFINITY) ? 0.0 : exp(mm - m);"),
    ("merge_drops_l", "l = l * sa + lb * sb;", "l = l + lb * sb;"),
    ("split_drops_key", "int64_t j0 = sp * len / ns, j1 = (sp + 1) * len / ns;",
     "int64_t j0 = sp * len / ns, j1 = (sp + 1) * len / ns - (sp + 1 < ns);"),
    ("seq_offset_shift", "off[b] = acc;", "off[b] = b ? acc - 1 : 0;"),
    ("max_not_updated", "if (sj > m) m = sj;", "if (sj > m && j == j0) m = sj;"),
    ("window_off_by_one", "j > p - window", "j >= p - window"),
    ("sink_inclusive", "(j < sink ||", "(j <= sink ||"),
    ("window_ignores_sink", "(j < sink || j > p - window)", "(j > p - window)"),
    ("window_from_row_index", "int64_t p = (int64_t)q_offset + t;", "int64_t p = (int64_t)t + (t > 0) * q_offset;"),
]

CHILD = textwrap.dedent("""
    import sys
    sys.path[:0] = [{root!r}, {tests!r}]
    from oracle import OracleLib
    import oracle_pins
    lib = OracleLib({lib!r})
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError) as e:
            caught.append(pin.__name__)
    print("CAUGHT", ",".join(caught))
""")


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert old in src, f"mutation site for {name} not found in the oracle source"
    path_c = tmp_path / f"{name}.c"
    path_so = tmp_path / f"lib{name}.so"
    path_c.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(path_c),
                    "-o", str(path_so), "-lm"], check=True)
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=str(path_so))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300, env={**os.environ, "OMP_NUM_THREADS": "2"})
    if r.returncode != 0:
        # a crash is also a caught mistake (out-of-range reads), but say so
        assert "CAUGHT" not in r.stdout or r.stdout.split("CAUGHT", 1)[1].strip(), r.stderr
        return
    caught = r.stdout.split("CAUGHT", 1)[1].strip()
    assert caught, f"mutant {name} passed every pin"
