"""Pins of the oracle's Philox4x32-10 (Salmon et al., SC'11, section 3.2)."""

import os
import shutil
import subprocess

import numpy as np
import pytest
import scipy.stats

from oracle.philox import philox4x32_10, seed_key, uniforms, word_to_uniform

HERE = os.path.dirname(os.path.abspath(__file__))

# Known-answer vectors published with the Random123 library that accompanies
# the SC'11 paper: (counter, key) -> output, all words hex.
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_known_answers(ctr, key, out):
    assert tuple(int(w) for w in philox4x32_10(ctr, key)) == out


def test_uniform_mapping_grid():
    assert word_to_uniform(0) == 0.0
    assert word_to_uniform(0xFFFFFFFF) == 1 - 2 ** -24
    assert word_to_uniform(0x100) == 2 ** -24
    u = uniforms(12345, 3, 4)
    w = philox4x32_10([3, 4, 0, 0], seed_key(12345))
    assert u == (int(w[0] >> 8) * 2 ** -24, int(w[1] >> 8) * 2 ** -24)
    # exactly representable in float32
    assert np.float32(u[0]) == u[0] and np.float32(u[1]) == u[1]


def test_uniformity():
    rows = np.arange(1 << 16, dtype=np.uint64)
    ctr = np.stack([rows, np.full_like(rows, 7), 0 * rows, 0 * rows], axis=-1)
    w = philox4x32_10(ctr, seed_key(0x0123456789ABCDEF))
    for i in range(4):
        bins = np.bincount((w[:, i] >> 24).astype(np.int64), minlength=256)
        assert scipy.stats.chisquare(bins).pvalue > 1e-4


def _rocrand_ref(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("rocRAND headers or hipcc not available")
    exe = tmp_path / "philox_ref"
    src = os.path.join(HERE, "rocrand_philox_ref.cpp")
    r = subprocess.run([hipcc, "-O1", "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", src,
                        "-o", str(exe)], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("could not build the rocRAND reference: " + r.stderr[-400:])
    return exe


@pytest.mark.parametrize("seed", [0, 0x0000000200000007, 0xFEDCBA9876543210])
def test_matches_rocrand(tmp_path, seed):
    exe = _rocrand_ref(tmp_path)
    out = subprocess.run([str(exe), hex(seed), "9", "17"], capture_output=True, text=True, check=True).stdout
    n = 0
    for line in out.strip().splitlines():
        r, p, *ws = line.split()
        ref = tuple(int(x, 16) for x in ws)
        got = tuple(int(x) for x in philox4x32_10([int(r), int(p), 0, 0], seed_key(seed)))
        assert got == ref, (r, p)
        n += 1
    assert n == 9 * 17
