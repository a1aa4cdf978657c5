"""Pins for the oracle's random numbers (Philox4x32-10, uniforms, Gumbel noise)."""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

TORCH_INC = None
try:
    import torch.utils.cpp_extension as _ce

    TORCH_INC = _ce.include_paths()[0]
except Exception:  # pragma: no cover
    pass


@pytest.fixture(scope="module")
def torch_philox(tmp_path_factory):
    """Build the PyTorch-header Philox reference (an implementation independent of ours)."""
    if TORCH_INC is None or shutil.which("g++") is None:
        pytest.skip("torch headers or g++ unavailable")
    src = os.path.join(os.path.dirname(__file__), "philox_torch_ref.cpp")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    subprocess.check_call(["g++", "-O1", "-std=c++17", "-I", TORCH_INC, src, "-o", exe])

    def run(blocks):
        inp = "\n".join(" ".join(str(int(v)) for v in b) for b in blocks) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True)
        return np.array([[int(t) for t in line.split()] for line in out.stdout.splitlines()],
                        dtype=np.uint64)

    return run


def test_philox_matches_independent_implementation(ora, torch_philox):
    rng = np.random.default_rng(123)
    blocks = [(0, 0, 0, 0, 0, 0), (0xFFFFFFFF,) * 6, (1, 2, 3, 4, 5, 6)]
    blocks += [tuple(int(v) for v in rng.integers(0, 2**32, 6, dtype=np.uint64))
               for _ in range(300)]
    ref = torch_philox(blocks)
    mine = np.array([ora.philox(b[:4], b[4:]) for b in blocks], dtype=np.uint64)
    assert np.array_equal(mine, ref)


def test_counter_layout(ora):
    # convention: key = (seed lo, seed hi); counter = (i>>2, r, k, cycle<<4 | stream)
    seed, cycle, stream, r, k = 0x0123456789ABCDEF, 77, 5, 9, 3
    for i in range(0, 12):
        block = ora.philox([i >> 2, r, k, (cycle << 4) | stream],
                           [seed & 0xFFFFFFFF, seed >> 32])
        assert ora.rand_word(seed, cycle, stream, r, k, i) == int(block[i & 3])


def test_uniform_grid_and_range(ora):
    for i in range(2000):
        w = ora.rand_word(7, 1, 2, i, 4, 0)
        u = ora.uniform(7, 1, 2, i, 4, 0)
        m = u * 2**24
        assert m == int(m) and int(m) % 2 == 1 and 0.0 < u < 1.0
        assert int(m) == 2 * (w >> 9) + 1
        assert np.float32(u) == u  # exactly representable in fp32


def test_uniform_is_uniform(ora):
    us = np.array([ora.uniform(3, 0, 1, r, 1, i) for r in range(100) for i in range(400)])
    counts, _ = np.histogram(us, bins=50, range=(0, 1))
    assert stats.chisquare(counts).pvalue > 1e-4


def test_gumbel_law(ora):
    g = np.array([ora.gumbel(11, 2, 0, r, 2, i) for r in range(100) for i in range(300)])
    assert stats.kstest(g, stats.gumbel_r.cdf).pvalue > 1e-4
    # bounded by the 24-bit uniform grid
    lo = -np.log(-np.log(2.0**-24))
    hi = -np.log(-np.log(1 - 2.0**-24))
    assert g.min() >= lo - 1e-12 and g.max() <= hi + 1e-12
