"""Pins for the oracle's Philox4x32-10 stream (CPU only).

Stochastic rounding of gradients is part of the recipe (readjensen.com NVFP4
training-recipe page, recipe paragraph; "Mastering Low-Precision AI", third
paragraph).  The generator is Philox4x32-10 (Salmon et al., SC'11).  The
oracle's implementation is checked against rocRAND's independent header
implementation, compiled here for the host, and by statistical checks.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    inc = "/opt/rocm/include"
    if not os.path.exists(os.path.join(inc, "rocrand", "rocrand_philox4x32_10.h")):
        pytest.skip("rocRAND headers not present")
    if shutil.which("g++") is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    subprocess.run(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I" + inc,
                    os.path.join(HERE, "rocrand_philox_ref.cpp"), "-o", exe], check=True)

    def run(queries):
        inp = "".join("%d %d %d\n" % q for q in queries)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [list(map(int, line.split())) for line in out.strip().splitlines()]
    return run


def test_philox_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(7)
    queries, ours = [], []
    cases = [(0, 0, 0), (1, 0, 0), (1, 1, 0), (1, 0, 1), (0xDEADBEEFCAFEF00D, 3, 12345),
             (2 ** 64 - 1, 2 ** 32 - 1, 2 ** 40 + 7), (42, 7, 2 ** 32 - 1), (42, 7, 2 ** 32)]
    for _ in range(200):
        cases.append((int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 32)),
                      int(rng.integers(0, 2 ** 60))))
    for seed, stream, g in cases:
        queries.append((seed, stream, 4 * g))
        ours.append(list(oracle.philox4x32_10(
            [g & 0xFFFFFFFF, (g >> 32) & 0xFFFFFFFF, stream, 0],
            [seed & 0xFFFFFFFF, seed >> 32])))
    assert rocrand_ref(queries) == ours


def test_sr_word_indexing(rocrand_ref):
    # element idx uses word idx & 3 of the block at counter idx >> 2
    seed, stream = 1, 1
    idxs = [0, 1, 2, 3, 4, 5, 1023, 2 ** 33 + 6]
    ref = rocrand_ref([(seed, stream, 4 * (i >> 2)) for i in idxs])
    for i, words in zip(idxs, ref):
        assert oracle.sr_word(seed, stream, i) == words[i & 3]


def test_sr_words_are_uniform_and_streams_differ():
    n = 1 << 14
    w0 = np.array([oracle.sr_word(1, 0, i) for i in range(n)], dtype=np.uint64)
    w1 = np.array([oracle.sr_word(1, 1, i) for i in range(n)], dtype=np.uint64)
    # each bit is set about half the time (4.5 sigma band)
    bits = ((w0[:, None] >> np.arange(32, dtype=np.uint64)[None, :]) & 1).mean(axis=0)
    assert np.all(np.abs(bits - 0.5) < 4.5 * 0.5 / np.sqrt(n))
    # chi-square of the top byte over 256 cells (dof 255; p ~ 1e-6 cut)
    hist = np.bincount((w0 >> 24).astype(np.int64), minlength=256)
    chi2 = ((hist - n / 256) ** 2 / (n / 256)).sum()
    assert chi2 < 380
    # the two streams are uncorrelated
    u0, u1 = w0 / 2.0 ** 32 - 0.5, w1 / 2.0 ** 32 - 0.5
    corr = (u0 * u1).mean() / np.sqrt((u0 ** 2).mean() * (u1 ** 2).mean())
    assert abs(corr) < 4.5 / np.sqrt(n)
    assert not np.array_equal(w0, w1)
