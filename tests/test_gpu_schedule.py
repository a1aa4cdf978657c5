"""GPU scheduler (dspark_schedule) against the oracle: ell, a and stats bit-exact in every
mode, on workload-shaped and adversarial confidences."""
import numpy as np
import pytest

from draft_sampling_scheduling_amd import synth
from tests.sched_sets import _conf_sets, _sps
from tests.gpu_util import N, T

pytestmark = pytest.mark.gpu
MODES = (0, 1, 2)


@pytest.fixture(scope="module")
def ds():
    import draft_sampling_scheduling_amd as ds
    ds.lib()
    return ds


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", range(7))
def test_schedule_bit_exact(ora, ds, mode, case):
    name, c, _, kind = _conf_sets()[case]
    R, gamma = c.shape
    sps, B0 = _sps(kind, R, gamma)
    c_lag = None
    if mode == 2:
        rng = np.random.default_rng(case)
        # the lagged batch must lie inside the table: workload tables start at B = R
        Rl = R if kind in ("c3", "c4") else max(1, R - 3)
        c_lag = np.clip(c[:Rl] + rng.normal(0, 0.05, (Rl, gamma)), 0, 1).astype(np.float32)
    o = ora.schedule(c, sps, B0, mode, c_lag=c_lag)
    g = ds.schedule(T(c), T(sps), B0, mode, c_lag=None if c_lag is None else T(c_lag))
    g = {k: N(v) for k, v in g.items()}
    assert np.array_equal(g["a"].view(np.uint32), o["a"].view(np.uint32)), name
    assert np.array_equal(g["ell"], o["ell"]), (name, np.nonzero(g["ell"] != o["ell"]))
    assert np.array_equal(g["stats"].view(np.uint64), o["stats"].view(np.uint64)), (name, g["stats"], o["stats"])


def test_confidence_fault_bit(ds):
    import torch
    c = np.full((4, 3), 0.5, np.float32)
    c[2, 1] = np.nan
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    sps = np.ones(16, np.float32)
    ds.schedule(T(c), T(sps), 1, 0, status=status)
    assert int(N(status)[0]) & ds.FAULT_CONF


@pytest.mark.parametrize("mode", MODES)
def test_schedule_deterministic(ds, mode):
    """Three runs on the same confidences give bit-identical lengths, survival and stats."""
    name, c, _, kind = _conf_sets()[4]  # the largest set (512 x 16)
    R, gamma = c.shape
    sps, B0 = _sps(kind, R, gamma)
    c_lag = c if mode == 2 else None
    runs = []
    for _ in range(3):
        g = ds.schedule(T(c), T(sps), B0, mode, c_lag=None if c_lag is None else T(c_lag))
        runs.append({k: N(v).tobytes() for k, v in g.items()})
    assert runs[0] == runs[1] == runs[2], name
