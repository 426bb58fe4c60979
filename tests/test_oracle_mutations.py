"""Plausible mistakes planted in copies of the oracle must each fail a pin.

Each mutant is built from lora_oracle.c with one textual change and run in a
subprocess (a mutant may read out of bounds), never touching the real oracle.
"""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "transposed_A": ("((int64_t)i * r + j) * d_in + c", "((int64_t)i * d_in + c) * r + j", 1),
    "transposed_B": ("((int64_t)i * d_out + o) * r + j", "((int64_t)i * r + j) * d_out + o", 1),
    "dropped_scale": ("acc[o] += sc * sum;", "acc[o] += sum;", 1),
    "wrong_sign": ("acc[o] += sc * sum;", "acc[o] -= sc * sum;", 1),
    "dropped_base": ("hit ? y0 + acc[o] : y0", "hit ? acc[o] : y0", 1),
    "minus1_touches": ("if (i == -1) continue;\n                hit = 1;", "hit = 1;\n                if (i == -1) continue;", 1),
    "first_slot_only": ("for (int k = 0; k < K; ++k) {\n                int i = (s >= 0)", "for (int k = 0; k < 1; ++k) {\n                int i = (s >= 0)", 1),
    "short_d_in": ("for (int c = 0; c < d_in; ++c)", "for (int c = 0; c < d_in - 1; ++c)", 1),
    "short_rank": ("for (int j = 0; j < ri; ++j)\n                        sum += v[j]", "for (int j = 1; j < ri; ++j)\n                        sum += v[j]", 1),
    "segment_off_by_one": ("for (int t = seg_off[s]; t < seg_off[s + 1]; ++t) owner[t] = s;", "for (int t = seg_off[s] + 1; t < seg_off[s + 1]; ++t) owner[t] = s;", 1),
    "row_uses_request": ("elem(x, dtype, (int64_t)t * ldx + c) *\n                               elem(A", "elem(x, dtype, (int64_t)s * ldx + c) *\n                               elem(A", 1),
    "shrink_drops_scale": ("vk[j] = sc * sum;", "vk[j] = sum;", 1),
    "expand_slot_offset": ("(int64_t)k * r + j] *", "(int64_t)k + j] *", 1),
    "merge_transposed_A": ("elem(A, dtype, ((int64_t)i * r + j) * d_in + c);\n                delta",
                           "elem(A, dtype, ((int64_t)i * d_in + c) * r + j);\n                delta", 1),
    "merge_drops_scale": ("delta += (scale ? (double)scale[k] : 1.0) * sum;", "delta += sum;", 1),
    "merge_ignores_alpha": ("+ alpha * delta;", "+ delta;", 1),
    "merge_uses_minus1": ("const int i = idx[k];\n                if (i == -1) continue;",
                          "int i = idx[k];\n                if (i == -1) i = 0;", 1),
    "ranks_ignored_in_apply": ("const int ri = ranks ? ranks[i] : r;  /* the adapter's own rank */",
                               "const int ri = r;", 1),
    "ranks_ignored_in_expand": ("const int ri = ranks ? ranks[i] : r;\n                double sum",
                                "const int ri = r;\n                double sum", 1),
    "merge_first_slot_only": ("for (int k = 0; k < K; ++k) {\n                const int i = idx[k];",
                              "for (int k = 0; k < 1; ++k) {\n                const int i = idx[k];", 1),
}

RUNNER = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, _pins
orc = oracle.Oracle({lib!r})
failed = _pins.run_all(orc)
print("FAILED:" + ",".join(failed))
"""


def _build_mutant(tmp, name, old, new, count):
    src = open(oracle.SRC).read()
    assert src.count(old) >= count, f"mutation {name}: pattern not found"
    mutated = src.replace(old, new, count)
    assert mutated != src
    path = os.path.join(tmp, f"{name}.c")
    open(path, "w").write(mutated)
    lib = os.path.join(tmp, f"lib{name}.so")
    oracle.build(src=path, out=lib)
    return lib


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new, count = MUTANTS[name]
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build_mutant(tmp, name, old, new, count)
        code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
        res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
        caught = res.returncode != 0 or ("FAILED:" in res.stdout and res.stdout.strip().split("FAILED:")[1] != "")
        assert caught, f"mutant {name} passed every pin:\n{res.stdout}\n{res.stderr}"
