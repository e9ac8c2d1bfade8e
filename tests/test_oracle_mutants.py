"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant is a one-token edit of ``oracle/hca_oracle.c`` of the kind a
careful reader could still miss (an off-by-one boundary, a flipped sign, a
dropped term, a swapped operand).  The copy is compiled to a temporary
library and the pin suite runs against it in a subprocess; the test passes
only if that run fails.  The real oracle source is never modified.

Two edits that look like mistakes are deliberately absent because they change
nothing (equivalent mutants): dropping STRICT mode's check that the whole
window lies in one document (a window that straddles a boundary only becomes
complete for queries past the boundary, whose document is not the window's
first), and dropping the "nominal rectangle" test in the tile classifier
(out-of-range elements already count as not visible).
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hca_oracle.c")

MUTANTS = {
    "completion_exclusive": ("if ((c + 1) * (int64_t)p->r > i + 1) return 0;",
                             "if ((c + 1) * (int64_t)p->r > i) return 0;"),
    "window_one_too_wide": ("if (!(i - p->W < t && t <= i)) return 0;",
                            "if (!(i - p->W <= t && t <= i)) return 0;"),
    "raw_sees_future": ("if (!(i - p->W < t && t <= i)) return 0;",
                        "if (!(i - p->W < t && t <= i + 1)) return 0;"),
    "no_raw_segment_check": ("  return seg_of(p, b, t) == seg_of(p, b, i);\n}",
                             "  return 1;\n}"),
    "last_mode_uses_first": ("if (p->comp_mode == 1) return seg_of(p, b, last);",
                             "if (p->comp_mode == 1) return seg_of(p, b, first);"),
    "strict_window_starts_late": ("int64_t first = (int64_t)c * p->r, last",
                                  "int64_t first = (int64_t)c * p->r + 1, last"),
    "delta_sign": ("double ds = s[k] * (dp[k] - dl);", "double ds = s[k] * (dp[k] + dl);"),
    "dq_unscaled": ("dq[d] += p->scale * ds * load_val(kb, p->in_dtype, koff + d);",
                    "dq[d] += ds * load_val(kb, p->in_dtype, koff + d);"),
    "dkv_drops_value_path": ("acc[d] += p->scale * dsk * load_val(q, p->in_dtype, qoff + d) +\n"
                             "                      pk * load_val(dout, p->in_dtype, qoff + d);",
                             "acc[d] += p->scale * dsk * load_val(q, p->in_dtype, qoff + d);"),
    "dkv_swaps_q_and_dout": ("acc[d] += p->scale * dsk * load_val(q, p->in_dtype, qoff + d) +\n"
                             "                      pk * load_val(dout, p->in_dtype, qoff + d);",
                             "acc[d] += p->scale * dsk * load_val(dout, p->in_dtype, qoff + d) +\n"
                             "                      pk * load_val(q, p->in_dtype, qoff + d);"),
    "lse_drops_max": ("if (lse) *lse = m + log(l);", "if (lse) *lse = log(l);"),
    "tile_rows_one_past": ("for (int64_t i = qt * bq; i < (qt + 1) * bq; ++i) {",
                           "for (int64_t i = qt * bq; i <= (qt + 1) * bq; ++i) {"),
    "tile_states_swapped": ("  return all ? 2 : 1;", "  return all ? 1 : 2;"),
    "mask_transposed": ("p->comp_mask[((int64_t)b * p->S + i) * p->Sc + c] != 0;",
                        "p->comp_mask[((int64_t)b * p->S + c) * p->Sc + i % p->Sc] != 0;"),
    "mask_mode_keeps_completion": ("  if (p->comp_mode == 2) return p->comp_mask[",
                                   "  if (p->comp_mode == 2 && (c + 1) * (int64_t)p->r <= i + 1)"
                                   " return p->comp_mask["),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {name}"
    mutated = tmp_path / "hca_oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w",
                           "-o", str(lib), str(mutated), "-lm"])
    env = dict(os.environ, HCA_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"mutant {name} passed every pin:\n{res.stdout[-2000:]}"
    assert "failed" in res.stdout, res.stdout[-2000:]
