"""The pins catch plausible mistakes in the oracle (CPU).  Each case plants
one mistake in a copy of oracle/kin_oracle.c (the tie-break, the
partial-block mean, the bf16 rounding, the softmax scale, the GQA sum, the
ranking direction, the token range of a block, the Quest bound, the
attended token range, the block count), builds it
with the oracle's own flags, and runs the pin suite against that build: at
least one pin must fail.  The planted mistakes live only in temporary
copies."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kin_oracle.c")
sys.path.insert(0, os.path.join(ROOT, "oracle"))
import build as oracle_build  # noqa: E402

MUTANTS = [
    ("tie-break-to-higher-index",
     "return (a->j > b->j) - (a->j < b->j);",
     "return (a->j < b->j) - (a->j > b->j);"),
    ("partial-block-mean-over-full-block",
     "double mean = sum / (double)n;",
     "double mean = sum / (double)c->block;"),
    ("bf16-ties-away-from-zero",
     "if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u)))",
     "if (drop >= 0x8000u)"),
    ("no-softmax-scale",
     "const double scale = 1.0 / sqrt((double)c->d);",
     "const double scale = 1.0;"),
    ("gqa-first-head-only",
     "for (int h = g * c->gqa; h < (g + 1) * c->gqa; ++h) {\n"
     "            size_t qo = ((size_t)b * hq + h) * c->d;\n"
     "            size_t so = ((size_t)pair * c->nb_cap + j) * c->d;",
     "for (int h = g * c->gqa; h < g * c->gqa + 1; ++h) {\n"
     "            size_t qo = ((size_t)b * hq + h) * c->d;\n"
     "            size_t so = ((size_t)pair * c->nb_cap + j) * c->d;"),
    ("lowest-scores-kept",
     "if (a->s > b->s)\n        return -1;\n    if (a->s < b->s)\n        return 1;",
     "if (a->s < b->s)\n        return -1;\n    if (a->s > b->s)\n        return 1;"),
    ("block-skips-first-token",
     "for (int t = t0; t < t0 + n; ++t) /* ascending token order */",
     "for (int t = t0 + 1; t < t0 + n; ++t) /* ascending token order */"),
    ("quest-bound-takes-minimum",
     "sigma += a > e ? a : e;",
     "sigma += a < e ? a : e;"),
    ("newest-token-not-attended",
     "t < (sel[i] + 1) * c->block && t < c->ctx_len; ++t)",
     "t < (sel[i] + 1) * c->block && t < c->ctx_len - 1; ++t)"),
    ("block-count-rounded-down",
     "static int kor_nblocks(int len, int block) { return (len + block - 1) / block; }",
     "static int kor_nblocks(int len, int block) { return len / block > 0 ? len / block : 1; }"),
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant, tmp_path):
    name, find, repl = mutant
    text = open(SRC).read()
    assert text.count(find) == 1, f"mutation site of {name} not found once"
    src = tmp_path / "kin_oracle.c"
    src.write_text(text.replace(find, repl))
    lib = tmp_path / "libkin_oracle.so"
    subprocess.run(["gcc", *oracle_build.CFLAGS, str(src), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, KIN_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"no pin fails with the planted mistake {name}:\n{r.stdout[-2000:]}"
