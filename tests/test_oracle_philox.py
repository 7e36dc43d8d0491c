"""Pin of the oracle's Philox-4x32-10 (oracle/attention.py) against rocRAND's.

The dropout keep mask is built from Philox-4x32-10 (Salmon, Moraes, Dror,
Shaw, SC 2011); the pages print no random numbers. The oracle writes the
generator from its published definition; this test compares its block
function, word for word, with the one of rocRAND (the ROCm random-number
library, an independent implementation shipped in the image as a header),
reached through the small host program tests/philox_ref.cpp, on 300 random
counters and keys plus the all-zero and all-ones words. A planted mistake in
the oracle's copy (one round fewer, a multiplier's bit flipped, the key
schedule's increments swapped) must be caught by the same comparison.

CPU only: the helper is host code built with hipcc (no GPU needed)."""
import inspect
import os
import shutil
import subprocess
import types

import numpy as np
import pytest

import oracle.attention as att

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    r = subprocess.run([HIPCC, "-O1", os.path.join(HERE, "philox_ref.cpp"), "-o", exe],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]

    def run(cases):
        inp = "\n".join(" ".join(str(int(x)) for x in row) for row in cases) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, timeout=120)
        assert out.returncode == 0
        return [[int(x) for x in line.split()] for line in out.stdout.strip().split("\n")]
    return run


def _cases():
    rng = np.random.default_rng(20261202)
    cases = rng.integers(0, 2 ** 32, size=(302, 6), dtype=np.uint64)
    cases[0] = 0
    cases[1] = 2 ** 32 - 1
    return cases


def _words(philox, cases):
    out = []
    for row in cases:
        w = philox(*[int(x) for x in row[:4]], int(row[4]), int(row[5]))
        out.append([int(np.asarray(x).item()) for x in w])
    return out


def test_oracle_philox_equals_rocrand(rocrand_philox):
    cases = _cases()
    assert _words(att.philox4x32_10, cases) == rocrand_philox(cases)


SRC = inspect.getsource(att)
MUTANTS = {
    "nine_rounds": ("for _ in range(10):", "for _ in range(9):"),
    "swapped_increments": ("k0 = (k0 + np.uint64(_PHILOX_W[0]))", "k0 = (k0 + np.uint64(_PHILOX_W[1]))"),
}


def _mutant(old, new):
    assert old in SRC, old
    mod = types.ModuleType("attention_mutant")
    exec(compile(SRC.replace(old, new), "attention_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(rocrand_philox, name):
    cases = _cases()[:40]
    assert _words(_mutant(*MUTANTS[name]).philox4x32_10, cases) != rocrand_philox(cases)


def test_flipped_multiplier_bit_is_caught(rocrand_philox):
    mod = _mutant("for _ in range(10):", "for _ in range(10):")
    mod._PHILOX_M = (mod._PHILOX_M[0] ^ 1,) + tuple(mod._PHILOX_M[1:])
    cases = _cases()[:40]
    assert _words(mod.philox4x32_10, cases) != rocrand_philox(cases)
