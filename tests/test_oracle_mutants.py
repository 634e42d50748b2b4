"""CPU-only: the pins must reject deliberately broken copies of the CPU reference.

Each mutant is oracle.c with one plausible mistake planted (a dropped term, a
wrong sign, index or operand), compiled into a temporary library and run
through every pin in a child process.  A mutant survives only if all pins
pass; none may survive.  The unmodified source must pass them all.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text to find, replacement, which occurrence (0-based))
MUTANTS = [
    ("dot_sign", "dot += q[d] * K[(int64_t)j * D + d];", "dot -= q[d] * K[(int64_t)j * D + d];", 0),
    ("drop_scale", "x[j] = scale * dot;", "x[j] = dot;", 0),
    ("lse_drop_max", "*lse = m + log(l);", "*lse = log(l);", 0),
    ("no_normalise", "out[d] = acc / l;", "out[d] = acc;", 0),
    ("no_max_shift", "x[j] = exp(x[j] - m);", "x[j] = exp(x[j]);", 0),
    ("pv_uses_k", "acc += x[j] * V[(int64_t)j * D + d];", "acc += x[j] * K[(int64_t)j * D + d];", 0),
    ("bf16_shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;", 0),
    ("gqa_map_decode", "int h = g * G + hh;", "int h = hh * H_kv + g;", 0),
    ("gqa_map_prefill", "int h = g * G + hh;", "int h = hh * H_kv + g;", 1),
    ("q_transposed", "const uint16_t *qr = &q[((int64_t)r * H_q + h) * D];",
     "const uint16_t *qr = &q[((int64_t)h * B + r) * D];", 0),
    ("drop_last_key", "int n = (s == 0 || hi <= lo) ? 0 : hi - lo;",
     "int n = (s == 0 || hi <= lo) ? 0 : hi - lo - 1;", 0),
    ("slot0_not_padding", "int n = (s == 0 || hi <= lo) ? 0 : hi - lo;",
     "int n = (hi <= lo) ? 0 : hi - lo;", 0),
    ("page_offset", "int64_t row = (int64_t)page * page_size + j % page_size;",
     "int64_t row = (int64_t)page * page_size + (j + 1) % page_size;", 0),
    ("block_index", "int page = page_table[(int64_t)s * max_blocks + j / page_size];",
     "int page = page_table[(int64_t)s * max_blocks + j / (2 * page_size)];", 1),
    ("prefill_not_causal", "softmax_attend(qd, K, V, i + 1, D, scale, x,",
     "softmax_attend(qd, K, V, n, D, scale, x,", 0),
    ("prefill_doc_base", "K[(int64_t)i * D + dd] = bf16_to_f64(k[((int64_t)(start + i) * H_kv + g) * D + dd]);",
     "K[(int64_t)i * D + dd] = bf16_to_f64(k[((int64_t)(i) * H_kv + g) * D + dd]);", 0),
    ("merge_weight", "double w = exp(ls - L);", "double w = exp(ls - M);", 0),
    ("merge_lse", "double L = M + log(sum);", "double L = log(sum);", 0),
    ("append_offset", "int64_t row = (int64_t)page * page_size + p % page_size;",
     "int64_t row = (int64_t)page * page_size + (p + 1) % page_size;", 0),
    ("append_page0", "if (page <= 0 || page >= num_pages) continue;",
     "if (page < 0 || page >= num_pages) continue;", 0),
]

_RUNNER = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle
oracle.use_library({lib!r})
from oracle_pins import ALL_PINS
for pin in ALL_PINS:
    try:
        pin()
    except AssertionError:
        print("killed by", pin.__name__)
        sys.exit(3)
sys.exit(0)
"""


def _mutate(text, find, repl, occ):
    start = -1
    for _ in range(occ + 1):
        start = text.find(find, start + 1)
        assert start >= 0, f"mutation site not found: {find!r} #{occ}"
    return text[:start] + repl + text[start + len(find):]


def _run_with(src_text, tmp, name):
    c = os.path.join(tmp, f"{name}.c")
    so = os.path.join(tmp, f"lib{name}.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", c, "-o", so, "-lm"],
                   check=True, capture_output=True)
    code = _RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=so)
    env = dict(os.environ, OMP_NUM_THREADS="2")
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=300)
    return p.returncode, p.stdout + p.stderr


def test_unmodified_copy_passes():
    with open(SRC) as f:
        text = f.read()
    with tempfile.TemporaryDirectory() as tmp:
        rc, out = _run_with(text, tmp, "clean")
    assert rc == 0, out


def test_every_mutant_is_killed():
    with open(SRC) as f:
        text = f.read()
    with tempfile.TemporaryDirectory() as tmp:
        def job(m):
            name, find, repl, occ = m
            rc, out = _run_with(_mutate(text, find, repl, occ), tmp, name)
            return name, rc, out

        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(job, MUTANTS))
    survivors = [(n, out[-300:]) for n, rc, out in results if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"


if __name__ == "__main__":  # pragma: no cover
    pytest.main([__file__, "-q"])
