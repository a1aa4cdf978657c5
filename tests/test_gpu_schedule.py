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


@pytest.mark.parametrize("fill", ["zeros", "ones", "random", "reused"])
def test_schedule_any_workspace_contents(ora, ds, fill):
    """The workspace needs no preparation: whatever it holds (zeros, all bits set, random
    bytes, or the state a call of another shape left), every mode gives the oracle's result,
    also on the next call with the same workspace."""
    import torch
    sets = _conf_sets()
    ws = torch.empty(ds.schedule_workspace_bytes(512, 16), dtype=torch.uint8, device="cuda:0")
    if fill == "zeros":
        ws.zero_()
    elif fill == "ones":
        ws.fill_(255)
    elif fill == "random":
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, generator=torch.Generator().manual_seed(5)))
    else:
        name, c, _, kind = sets[4]  # 512 x 16
        sps, B0 = _sps(kind, *c.shape)
        ds.schedule(T(c), T(sps), B0, ds.GLOBAL, ws=ws)
    for case in (0, 6, 1):
        name, c, _, kind = sets[case]
        R, gamma = c.shape
        sps, B0 = _sps(kind, R, gamma)
        for mode in MODES:
            c_lag = None
            if mode == 2:
                Rl = R if kind in ("c3", "c4") else max(1, R - 3)
                c_lag = np.clip(c[:Rl] * 0.97, 0, 1).astype(np.float32)
            o = ora.schedule(c, sps, B0, mode, c_lag=c_lag)
            g = ds.schedule(T(c), T(sps), B0, mode, c_lag=None if c_lag is None else T(c_lag),
                            ws=ws)
            g = {k: N(v) for k, v in g.items()}
            assert np.array_equal(g["ell"], o["ell"]), (fill, name, mode)
            assert np.array_equal(g["stats"].view(np.uint64), o["stats"].view(np.uint64)), (fill, name, mode)


@pytest.mark.parametrize("mode", MODES)
def test_schedule_graph_replays(ora, ds, mode):
    """The call captured once in a HIP graph and replayed with new confidences copied into
    its input between replays (eager work and synchronisation in between): every replay
    gives the oracle's result for the confidences it saw."""
    import torch
    rng = np.random.default_rng(11 + mode)
    name, c0, _, kind = _conf_sets()[0]  # 256 x 8, the workload's shape
    R, gamma = c0.shape
    sps, B0 = _sps(kind, R, gamma)
    dev = torch.device("cuda:0")
    c_buf = T(c0)
    lag_buf = T(c0) if mode == 2 else None
    sps_t = T(sps)
    out = dict(ell=torch.empty(R, dtype=torch.int32, device=dev),
               a=torch.empty((R, gamma), dtype=torch.float32, device=dev),
               stats=torch.empty(4, dtype=torch.float64, device=dev))
    ws = torch.empty(ds.schedule_workspace_bytes(R, gamma), dtype=torch.uint8, device=dev)
    ds.schedule(c_buf, sps_t, B0, mode, c_lag=lag_buf, out=out, ws=ws)  # first call outside
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ds.schedule(c_buf, sps_t, B0, mode, c_lag=lag_buf, out=out, ws=ws)
    for rep in range(4):
        c = rng.beta(6, 1.6, (R, gamma)).astype(np.float32)
        c_buf.copy_(T(c))
        c_lag = None
        if mode == 2:
            c_lag = np.clip(c * rng.uniform(0.9, 1.0), 0, 1).astype(np.float32)
            lag_buf.copy_(T(c_lag))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o = ora.schedule(c, sps, B0, mode, c_lag=c_lag)
        assert np.array_equal(N(out["ell"]), o["ell"]), (mode, rep)
        assert np.array_equal(N(out["stats"]).view(np.uint64), o["stats"].view(np.uint64)), (mode, rep)


SHAPES = [(1, 1, None), (1, 64, None), (4096, 1, None), (4097, 1, None), (8192, 1, None),
          (128, 64, None), (37, 7, 74), (300, 9, 5)]


@pytest.mark.parametrize("R,gamma,R_lag", SHAPES)
def test_schedule_shape_edges(ora, ds, R, gamma, R_lag):
    """Shapes at the kernel's edges: one entry, one request with 64 positions, the entry
    counts around the change from one to two entries per wave (4096 / 4097) and the largest
    (8192, as 8192 x 1 and 128 x 64), and lagged batches larger and smaller than the current
    one; every mode bit-exact against the oracle."""
    rng = np.random.default_rng(R * 131 + gamma)
    c = rng.beta(5, 1.5, (R, gamma)).astype(np.float32)
    c[rng.random((R, gamma)) < 0.02] = 1.0
    Rmax = max(R, R_lag or 0)
    B = np.arange(1, Rmax * (gamma + 1) + 1, dtype=np.float64)
    sps = (1.0 / (1.0 + 0.002 * B + 0.01 * np.floor(B / 29))).astype(np.float32)
    modes = MODES if R_lag is not None else (0, 1)
    for mode in modes:
        c_lag = None
        if mode == 2:
            c_lag = rng.beta(5, 1.5, (R_lag, gamma)).astype(np.float32)
        o = ora.schedule(c, sps, 1, mode, c_lag=c_lag)
        g = ds.schedule(T(c), T(sps), 1, mode, c_lag=None if c_lag is None else T(c_lag))
        g = {k: N(v) for k, v in g.items()}
        assert np.array_equal(g["ell"], o["ell"]), (R, gamma, mode)
        assert np.array_equal(g["a"].view(np.uint32), o["a"].view(np.uint32)), (R, gamma, mode)
        assert np.array_equal(g["stats"].view(np.uint64), o["stats"].view(np.uint64)), (R, gamma, mode)
