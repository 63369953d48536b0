"""Pins of the oracle's counter-based RNG (Philox4x32-10).

The pages ("Pretraining Large Language Models with NVFP4", Technische
Zusammenfassung 2.B.4) only ask for stochastic rounding of gradients; the
random source is a reading: Philox4x32-10 (Salmon et al., SC'11).  The oracle's
implementation is checked against rocRAND's philox4x32_10 engine, an
independent library implementation, built here for the host from its header.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROCRAND_INC = "/opt/rocm/include"


@pytest.fixture(scope="module")
def rocrand_philox(tmp_path_factory):
    if not os.path.exists(os.path.join(ROCRAND_INC, "rocrand", "rocrand_philox4x32_10.h")):
        pytest.skip("rocRAND headers not present")
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_check")
    subprocess.run([cxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", ROCRAND_INC,
                    os.path.join(HERE, "philox_rocrand_check.cpp"), "-o", exe], check=True)

    def run(rows):
        inp = "".join(" ".join(f"{v:08x}" for v in r) + "\n" for r in rows)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [[int(w, 16) for w in line.split()] for line in out.strip().splitlines()]

    return run


def test_philox_matches_rocrand(rocrand_philox):
    rng = np.random.default_rng(7)
    rows = [[0, 0, 0, 0, 0, 0], [0xFFFFFFFF] * 6, [0, 0, 0, 0, 0, 1]]
    rows += [list(map(int, rng.integers(0, 2 ** 32, 6, dtype=np.uint64))) for _ in range(3000)]
    rows += [[5, 0, i, 0, 0, 0] for i in range(1000)]
    want = rocrand_philox(rows)
    for r, w in zip(rows, want):
        got = oracle.philox4x32_10([r[2], r[3], r[4], r[5]], [r[0], r[1]])
        assert list(map(int, got)) == w, r


def test_sr_draw_layout():
    # element idx takes half (idx % 2) of word (idx % 8) // 2 of the block idx // 8
    seed = 0x123456789ABCDEF0
    key = [seed & 0xFFFFFFFF, seed >> 32]
    d = oracle.sr_draws(seed, 0, 64)
    for g in range(8):
        w = oracle.philox4x32_10([g, 0, 0, 0], key)
        for j in range(8):
            assert d[8 * g + j] == (int(w[j >> 1]) >> (16 * (j & 1))) & 0xFFFF
    # high counter word is used for large indices
    big = (1 << 35) + 3
    w = oracle.philox4x32_10([(big >> 3) & 0xFFFFFFFF, big >> 35, 0, 0], key)
    assert oracle.sr_draws(seed, big, 1)[0] == (int(w[1]) >> 16) & 0xFFFF


def test_rht_sign_mask_definition():
    for seed in [0, 1, 1000, 2 ** 40 + 5]:
        w = oracle.philox4x32_10([0, 0, 0, 1], [seed & 0xFFFFFFFF, seed >> 32])
        assert oracle.rht_sign_mask(seed) == int(w[0]) & 0xFFFF


def test_sr_draws_uniform():
    # chi-square over 256 bins of the high byte, 2^20 draws: far from the 1e-6 tails
    d = oracle.sr_draws(3, 0, 1 << 20)
    counts = np.bincount(d >> 8, minlength=256)
    exp = len(d) / 256
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert 150 < chi2 < 380
