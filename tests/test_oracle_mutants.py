"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case rewrites one expression of oracle/bsmm_oracle.c (a dropped term, a
transposed operand, a wrong index, sign or bias), builds that copy into a
temporary directory and runs the pins of pins.py against it; at least one pin
has to fail.  Every rewrite keeps all memory accesses in bounds.
"""
import os

import pytest

import oracle
import pins

MUTANTS = [
    ("fprop reads W transposed", "orc_decode(w, (id * b + i) * b + j, dt);",
     "orc_decode(w, (id * b + j) * b + i, dt);", 0),
    ("bprop reads W untransposed", "orc_decode(w, (id * b + i) * b + j, dt);",
     "orc_decode(w, (id * b + j) * b + i, dt);", 1),
    ("fprop drops the last input block", "for (int64_t c = 0; c < R; c++) {\n                    int64_t id",
     "for (int64_t c = 0; c < R - 1; c++) {\n                    int64_t id", 0),
    ("bprop drops the first output block", "for (int64_t k = 0; k < S; k++) {\n                    int64_t id",
     "for (int64_t k = 1; k < S; k++) {\n                    int64_t id", 0),
    ("feature_axis=0 indexed as feature_axis=1", "return fa ? n * F + f : f * N + n;",
     "return n * F + f;", 0),
    ("f16 exponent bias", "e - 25", "e - 24", 0),
    ("f16 subnormal scale", "ldexp((double)m, -24)", "ldexp((double)m, -23)", 0),
    ("bf16 shift", "<< 16", "<< 15", 0),
    ("grouped dW keeps only step 0", "for (int g = 0; g < G; g++)", "for (int g = 0; g < 1; g++)", 0),
    ("dW block stored transposed", "dw[(t * b + i) * b + j] = acc;", "dw[(t * b + j) * b + i] = acc;", 0),
    ("dW reads a reversed dy column", "act_index(fa, N, K, n, k * b + j), dt);\n",
     "act_index(fa, N, K, n, k * b + (b - 1 - j)), dt);\n", 0),
    ("fprop sign", "acc += orc_decode(x,", "acc -= orc_decode(x,", 0),
    ("identity on every block", "(c == k && i == j)", "(i == j)", 0),
    ("block ids numbered column-major",
     "    for (int64_t c = 0; c < R; c++)\n        for (int64_t k = 0; k < S; k++)\n            id_of[c * S + k]",
     "    for (int64_t k = 0; k < S; k++)\n        for (int64_t c = 0; c < R; c++)\n            id_of[c * S + k]", 0),
    ("block_coord off by one", "if (id == block)", "if (id == block + 1)", 0),
    ("fprop skips the last minibatch row", "for (int64_t n = 0; n < N; n++)\n            for (int64_t j",
     "for (int64_t n = 0; n < N - 1; n++)\n            for (int64_t j", 0),
    ("accumulator not cleared", "double acc = 0.0;", "double acc = 1e-3;", 1),
]


def _replace_nth(s, old, new, nth):
    start = -1
    for _ in range(nth + 1):
        start = s.find(old, start + 1)
        assert start >= 0, f"mutation target not found: {old!r}"
    return s[:start] + new + s[start + len(old):]


@pytest.mark.parametrize("name,old,new,nth", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new, nth):
    src = open(oracle.SRC).read()
    mutated = _replace_nth(src, old, new, nth)
    assert mutated != src
    csrc = os.path.join(tmp_path, "mutant.c")
    with open(csrc, "w") as f:
        f.write(mutated)
    lib = oracle.load(oracle.build(src=csrc, out=os.path.join(tmp_path, "libmutant.so")))
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, IndexError) as e:
            failed.append(pin.__name__)
            break
    assert failed, f"no pin caught the planted mistake: {name}"
