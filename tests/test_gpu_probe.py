"""dspark_read_probe, the benchmark's read-rate calibration: the XOR of its sink is the XOR
of every 32-bit word of the buffer, for grids that split the buffer evenly, raggedly, and
into more slices than it has 16-byte chunks (the surplus workgroups read nothing)."""
import numpy as np
import pytest

from tests.gpu_util import N, T

pytestmark = pytest.mark.gpu

CASES = [(4, 1), (4 * 777, 13), (1 << 20, 2048), (4 * 100, 4096), ((1 << 22) + 4 * 3, 1000)]


@pytest.mark.parametrize("nwords,grid", CASES, ids=[f"w{c[0]}-g{c[1]}" for c in CASES])
def test_read_probe_reads_every_word(nwords, grid):
    import draft_sampling_scheduling_amd as ds
    rng = np.random.default_rng(nwords + grid)
    a = rng.integers(0, 1 << 32, nwords, dtype=np.uint64).astype(np.uint32)
    sink = N(ds.read_probe(T(a.view(np.int32)), grid)).view(np.uint32)
    assert sink.shape == (grid,)
    assert np.bitwise_xor.reduce(sink) == np.bitwise_xor.reduce(a)
