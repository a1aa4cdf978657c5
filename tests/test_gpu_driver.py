"""GPU multi-cycle decode (dspark_decode_run) against the oracle's driver on the same toy
chain: every emitted token, the per-request counts and the per-position counters must be
identical, for each length policy (the scheduler's three modes, fixed length, static
threshold).  A token decided at a near-tie would diverge the sequences from there on; the
seeded chains here have none."""
import numpy as np
import pytest

from draft_sampling_scheduling_amd import synth
from tests.gpu_util import N, T, W2T

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ds():
    import draft_sampling_scheduling_amd as ds
    ds.lib()
    return ds


def _both(ora, ds, C, ncycles, policy, threshold=0.0, temps=None):
    o = ora.decode_run(C["Ub"], C["Hb"], C["W1"], C["W2"], C["w"], C["Tb"], C["x0"], ncycles,
                       policy=policy, threshold=threshold, sps=C["sps"], sps_B0=C["sps_B0"],
                       seed=11, temps=temps)
    W2t = W2T(C["W2"])
    g = ds.decode_run(T(C["Ub"]), T(C["Hb"]), T(C["W1"]), T(W2t), T(C["w"]), T(C["Tb"]),
                      T(C["x0"]), ncycles, policy=policy, threshold=threshold, sps=T(C["sps"]),
                      sps_B0=C["sps_B0"], seed=11, temps=None if temps is None else T(temps))
    return o, {k: N(v) for k, v in g.items()}


def _check(o, g, gamma, label):
    st = g["stats"]
    assert np.array_equal(g["n_emitted"], o["n_emitted"]), label
    for q in range(len(o["n_emitted"])):
        assert np.array_equal(g["tokens"][q], o["tokens"][q]), (label, q)
    assert np.array_equal(st[:gamma], o["tested"]), (label, st[:gamma], o["tested"])
    assert np.array_equal(st[gamma:2 * gamma], o["accepted"]), label
    assert [int(x) for x in st[2 * gamma:]] == [o["sum_ell"], o["emitted"], o["request_cycles"]]


CASES = [
    ("sync", 0, 0.0),
    ("global", 1, 0.0),
    ("async-lag2", 2, 0.0),
    ("fixed", 3, 0.0),
    ("threshold", 4, 0.3),
]


@pytest.mark.parametrize("name,policy,thr", CASES, ids=[c[0] for c in CASES])
def test_decode_parity(ora, ds, name, policy, thr):
    C = synth.toy_chain(V=1024, gamma=4, r=16, d=8, R=48, seed=2)
    print(f"{name}: R=48 gamma=4 V=1024, 8 cycles", flush=True)
    o, g = _both(ora, ds, C, 8, policy, thr)
    _check(o, g, 4, name)
    assert o["emitted"] > o["request_cycles"]  # some drafts were accepted


def test_decode_parity_wider(ora, ds):
    # r = 64, gamma = 8, a ragged vocabulary, calibrated temperatures
    C = synth.toy_chain(V=1000, gamma=8, r=64, d=16, R=20, seed=3)
    temps = np.linspace(0.8, 1.6, 8).astype(np.float32)
    print("wider: R=20 gamma=8 V=1000 r=64, 5 cycles", flush=True)
    o, g = _both(ora, ds, C, 5, 0, temps=temps)
    _check(o, g, 8, "wider")


def test_decode_zero_cycles_and_bad_anchor(ds):
    import torch
    C = synth.toy_chain(V=512, gamma=2, r=16, d=8, R=4, seed=4)
    W2t = W2T(C["W2"])
    args = [T(C["Ub"]), T(C["Hb"]), T(C["W1"]), T(W2t), T(C["w"]), T(C["Tb"])]
    g = ds.decode_run(*args, T(C["x0"]), 0, policy=3)
    assert N(g["n_emitted"]).sum() == 0 and N(g["stats"]).sum() == 0
    x0 = C["x0"].copy()
    x0[1] = 600
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    ds.decode_run(*args, T(x0), 2, policy=3, status=status)
    assert int(N(status)[0]) & ds.FAULT_TOKEN
