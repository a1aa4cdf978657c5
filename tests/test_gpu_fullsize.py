"""Parity at the full workload sizes, through the same entry points and launch
configuration bench.py times: the headline workload (R=256, gamma=8, V=151936, r=256,
d=4096, bf16) end to end (draft, schedule, verify), the RNN-head workload's draft
(R=256, gamma=16, V=129280) and the largest workload's draft (R=512, gamma=16, V=151936,
d=5120: U is 2.49 GB, near the 4 GiB reach of the sweep's 32-bit offsets, and every
workgroup takes two row groups).  The oracle runs the whole workload on the host (a few seconds
on the machine's cores); every request is compared by the same rules as the scaled tests."""
import numpy as np
import pytest

from draft_sampling_scheduling_amd import synth
from tests.gpu_util import N, T, compare_draft, compare_verify

pytestmark = pytest.mark.gpu

CYCLE = 3


@pytest.fixture(scope="module")
def ds():
    import draft_sampling_scheduling_amd as ds
    ds.lib()
    return ds


@pytest.fixture(scope="module")
def c3(ora):
    cfg = synth.CONFIGS["c3"]
    I = synth.inputs(cfg)
    d = ora.draft_markov(I["U"], I["h"], I["W1"], I["W2"], I["w"], I["x0"], 0, CYCLE)
    return cfg, I, d


def _gpu_draft(ds, cfg, I, rnn=False):
    W2t = np.ascontiguousarray(I["W2"].T)
    if rnn:
        g = ds.draft_rnn(T(I["U"]), T(I["h"]), T(I["W1"]), T(W2t), T(I["W_gco"]), T(I["w"]),
                         T(I["x0"]), 0, CYCLE)
    else:
        g = ds.draft_markov(T(I["U"]), T(I["h"]), T(I["W1"]), T(W2t), T(I["w"]), T(I["x0"]),
                            0, CYCLE)
    g = {k: N(v) for k, v in g.items()}
    if g["bias_rows"].dtype == np.uint16:
        g["bias_rows"] = synth.bf16_to_f32(g["bias_rows"])
    return g


def test_c3_draft_full(ora, ds, c3):
    cfg, I, o = c3
    print(f"c3 draft: R={cfg.R} gamma={cfg.gamma} V={cfg.V}", flush=True)
    g = _gpu_draft(ds, cfg, I)
    compared, excused = compare_draft(o, g, "c3-full")
    print(f"c3 draft: compared {compared}, excused {excused}")


def test_c3_schedule_full(ora, ds, c3):
    cfg, I, o = c3
    c = o["c"].astype(np.float32)
    sps = synth.sps_table(cfg)
    ref = ora.schedule(c, sps, cfg.sps_B0, 0)
    g = ds.schedule(T(c), T(sps), cfg.sps_B0, 0)
    assert np.array_equal(N(g["ell"]), ref["ell"])
    assert np.array_equal(N(g["a"]), ref["a"].astype(np.float32))


def test_c3_verify_full(ora, ds, c3):
    cfg, I, d = c3
    # target stand-in: the drafted logits plus noise; bonus row fresh (as the scaled tests)
    W2 = synth.decode(cfg, I["W2"]).astype(np.float32)
    logits = synth.decode(cfg, I["U"]).astype(np.float32)
    logits += np.matmul(d["bias_rows"].astype(np.float32), W2)
    noise, fresh = synth.target_parts(cfg, range(cfg.R), CYCLE)
    target = synth.encode(cfg, np.concatenate([logits, fresh[:, None, :]], axis=1) + noise)
    del logits, noise
    ell = ora.schedule(d["c"].astype(np.float32), synth.sps_table(cfg), cfg.sps_B0, 0)["ell"]
    print(f"c3 verify: {int(ell.sum())} verified rows", flush=True)
    o = ora.verify(target, I["U"], I["W2"], d["bias_rows"], d["x"], ell, seed=0, cycle=CYCLE)
    brows = synth.encode(cfg, d["bias_rows"].astype(np.float32))  # exact: rows of W1
    W2t = np.ascontiguousarray(I["W2"].T)
    g = ds.verify(T(target), T(I["U"]), T(W2t), T(brows), T(d["x"]),
                  T(d["lse"].astype(np.float32)), T(d["logit_x"].astype(np.float32)), T(ell),
                  seed=0, cycle=CYCLE)
    g = {k: N(v) for k, v in g.items()}
    excused = compare_verify(o, g, ell, "c3-full")
    print(f"c3 verify: accepted {int(o['n_acc'].sum())}, excused {excused}")


def test_c5_rnn_draft_full(ora, ds):
    cfg = synth.CONFIGS["c5"]
    I = synth.inputs(cfg)
    print(f"c5 draft: R={cfg.R} gamma={cfg.gamma} V={cfg.V}", flush=True)
    o = ora.draft_rnn(I["U"], I["h"], I["W1"], I["W2"], I["W_gco"], I["w"], I["x0"], 0, CYCLE)
    g = _gpu_draft(ds, cfg, I, rnn=True)
    compared, excused = compare_draft(o, g, "c5-full")
    print(f"c5 draft: compared {compared}, excused {excused}")


def test_c4_draft_full(ora, ds):
    cfg = synth.CONFIGS["c4"]
    I = synth.inputs(cfg)
    print(f"c4 draft: R={cfg.R} gamma={cfg.gamma} V={cfg.V} d={cfg.d}", flush=True)
    o = ora.draft_markov(I["U"], I["h"], I["W1"], I["W2"], I["w"], I["x0"], 0, CYCLE)
    g = _gpu_draft(ds, cfg, I)
    compared, excused = compare_draft(o, g, "c4-full")
    print(f"c4 draft: compared {compared}, excused {excused}")
