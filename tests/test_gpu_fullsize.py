"""Parity at the full workload sizes, through the same entry points and launch
configuration bench.py times:

  - the mid-size workload (R=64, gamma=8, V=32000, d=2560) end to end: draft, schedule
    (early stop), verify;
  - the headline workload (R=256, gamma=8, V=151936, r=256, d=4096, bf16) end to end;
  - the largest workload (R=512, gamma=16, V=151936, d=5120: U is 2.49 GB, near the 4 GiB
    reach of the sweep's 32-bit offsets, every workgroup takes two row groups): draft, the
    no-break schedule, and verify of its lengths (target logits 2.64 GB);
  - the RNN-head workload (R=256, gamma=16, V=129280) as one cycle of the production loop:
    the RNN draft of this cycle and of the cycle two before, the two-step-lag schedule on
    those confidences, verification with the float bias rows.
Each stage is compared with the oracle on identical inputs (the GPU stage's inputs), so a
near-tie upstream does not cascade; the oracle runs the whole workload on the host (seconds
to a minute on the host's cores)."""
import numpy as np
import pytest

from draft_sampling_scheduling_amd import synth
from tests.gpu_util import N, T, W2T, compare_draft, compare_verify

pytestmark = pytest.mark.gpu

CYCLE = 3


@pytest.fixture(scope="module")
def ds():
    import draft_sampling_scheduling_amd as ds
    ds.lib()
    return ds


def _oracle_draft(ora, cfg, I, cycle=CYCLE):
    if cfg.head == "rnn":
        return ora.draft_rnn(I["U"], I["h"], I["W1"], I["W2"], I["W_gco"], I["w"], I["x0"], 0,
                             cycle)
    return ora.draft_markov(I["U"], I["h"], I["W1"], I["W2"], I["w"], I["x0"], 0, cycle)


@pytest.fixture(scope="module")
def c3(ora):
    cfg = synth.CONFIGS["c3"]
    I = synth.inputs(cfg)
    return cfg, I, _oracle_draft(ora, cfg, I)


@pytest.fixture(scope="module")
def c4(ora):
    cfg = synth.CONFIGS["c4"]
    I = synth.inputs(cfg)
    print(f"c4: oracle draft R={cfg.R} gamma={cfg.gamma} V={cfg.V} d={cfg.d}", flush=True)
    return cfg, I, _oracle_draft(ora, cfg, I)


@pytest.fixture(scope="module")
def c5(ora):
    cfg = synth.CONFIGS["c5"]
    I = synth.inputs(cfg)
    print(f"c5: oracle RNN draft R={cfg.R} gamma={cfg.gamma} V={cfg.V}", flush=True)
    return cfg, I, _oracle_draft(ora, cfg, I)


def _gpu_draft(ds, cfg, I, cycle=CYCLE):
    W2t = W2T(I["W2"])
    if cfg.head == "rnn":
        g = ds.draft_rnn(T(I["U"]), T(I["h"]), T(I["W1"]), W2t, T(I["W_gco"]), T(I["w"]),
                         T(I["x0"]), 0, cycle)
    else:
        g = ds.draft_markov(T(I["U"]), T(I["h"]), T(I["W1"]), W2t, T(I["w"]), T(I["x0"]), 0,
                            cycle)
    g = {k: N(v) for k, v in g.items()}
    if g["bias_rows"].dtype == np.uint16:
        g["bias_rows"] = synth.bf16_to_f32(g["bias_rows"])
    return g


def _target(cfg, I, bias_rows, cycle=CYCLE, chunk=32):
    """Target stand-in for one cycle: the drafted logits U + bias W2 plus seeded noise for
    rows 1..gamma, a fresh U-law row plus noise for the bonus row; built in request chunks
    (encoded operand type)."""
    W2 = synth.decode(cfg, I["W2"]).astype(np.float32)
    out = np.empty((cfg.R, cfg.gamma + 1, cfg.V), np.uint16 if cfg.is_bf16 else np.float32)
    for q0 in range(0, cfg.R, chunk):
        qs = range(q0, min(cfg.R, q0 + chunk))
        logits = synth.decode(cfg, I["U"][q0:qs.stop]).astype(np.float32)
        logits += np.matmul(np.asarray(bias_rows[q0:qs.stop], np.float32), W2)
        noise, fresh = synth.target_parts(cfg, qs, cycle)
        out[q0:qs.stop] = synth.encode(cfg, np.concatenate([logits, fresh[:, None, :]], axis=1)
                                       + noise)
    return out


def _verify_both(ora, ds, cfg, I, target, x, lse, logit_x, bias_rows, ell, label,
                 cycle=CYCLE):
    """Oracle and GPU verification on the same drafted block; bias_rows as the GPU takes
    them (bf16 bits of W1 rows for the Markov head, float for the RNN head)."""
    print(f"{label}: {int(ell.sum())} verified rows", flush=True)
    br64 = (synth.bf16_to_f32(bias_rows) if bias_rows.dtype == np.uint16
            else bias_rows).astype(np.float64)
    o = ora.verify(target, I["U"], I["W2"], br64, x, ell, seed=0, cycle=cycle)
    g = ds.verify(T(target), T(I["U"]), W2T(I["W2"]), T(bias_rows), T(x),
                  T(lse.astype(np.float32)), T(logit_x.astype(np.float32)), T(ell), seed=0,
                  cycle=cycle)
    g = {k: N(v) for k, v in g.items()}
    excused = compare_verify(o, g, ell, label)
    print(f"{label}: accepted {int(o['n_acc'].sum())}, excused {excused}")
    return o, g


def _schedule_both(ora, ds, cfg, c, mode, c_lag=None):
    sps = synth.sps_table(cfg)
    c = np.asarray(c, np.float32)
    o = ora.schedule(c, sps, cfg.sps_B0, mode, c_lag=c_lag)
    g = ds.schedule(T(c), T(sps), cfg.sps_B0, mode, c_lag=None if c_lag is None else T(c_lag))
    g = {k: N(v) for k, v in g.items()}
    assert np.array_equal(g["ell"], o["ell"])
    assert np.array_equal(g["a"].view(np.uint32), o["a"].view(np.uint32))
    assert np.array_equal(g["stats"].view(np.uint64), o["stats"].view(np.uint64))
    return o["ell"]


def test_c2_cycle_full(ora, ds):
    cfg = synth.CONFIGS["c2"]
    I = synth.inputs(cfg)
    print(f"c2 cycle: R={cfg.R} gamma={cfg.gamma} V={cfg.V} d={cfg.d}", flush=True)
    o = _oracle_draft(ora, cfg, I)
    g = _gpu_draft(ds, cfg, I)
    compare_draft(o, g, "c2-full")
    ell = _schedule_both(ora, ds, cfg, g["c"], ora.SYNC_BREAK)
    brows = synth.encode(cfg, g["bias_rows"])  # exact: rows of W1
    target = _target(cfg, I, g["bias_rows"])
    _verify_both(ora, ds, cfg, I, target, g["x"], g["lse"], g["logit_x"], brows, ell,
                 "c2-full")


def test_c3_draft_full(ora, ds, c3):
    cfg, I, o = c3
    print(f"c3 draft: R={cfg.R} gamma={cfg.gamma} V={cfg.V}", flush=True)
    g = _gpu_draft(ds, cfg, I)
    compared, excused = compare_draft(o, g, "c3-full")
    print(f"c3 draft: compared {compared}, excused {excused}")


def test_c3_schedule_full(ora, ds, c3):
    cfg, I, o = c3
    _schedule_both(ora, ds, cfg, o["c"], ora.SYNC_BREAK)


def test_c3_verify_full(ora, ds, c3):
    cfg, I, d = c3
    ell = ora.schedule(d["c"].astype(np.float32), synth.sps_table(cfg), cfg.sps_B0, 0)["ell"]
    brows = synth.encode(cfg, d["bias_rows"].astype(np.float32))  # exact: rows of W1
    target = _target(cfg, I, d["bias_rows"])
    _verify_both(ora, ds, cfg, I, target, d["x"], d["lse"], d["logit_x"], brows, ell,
                 "c3-full")


def test_c4_draft_full(ora, ds, c4):
    cfg, I, o = c4
    g = _gpu_draft(ds, cfg, I)
    compared, excused = compare_draft(o, g, "c4-full")
    print(f"c4 draft: compared {compared}, excused {excused}")


def test_c4_schedule_and_verify_full(ora, ds, c4):
    """The no-break search (the workload's scheduler) on the drafted confidences, then
    verification of those lengths at R=512, gamma=16, V=151936."""
    cfg, I, d = c4
    ell = _schedule_both(ora, ds, cfg, d["c"], ora.GLOBAL)
    assert ell.sum() > 0
    brows = synth.encode(cfg, d["bias_rows"].astype(np.float32))  # exact: rows of W1
    target = _target(cfg, I, d["bias_rows"])
    _verify_both(ora, ds, cfg, I, target, d["x"], d["lse"], d["logit_x"], brows, ell,
                 "c4-full")


def test_c5_rnn_draft_full(ora, ds, c5):
    cfg, I, o = c5
    print(f"c5 draft: R={cfg.R} gamma={cfg.gamma} V={cfg.V}", flush=True)
    g = _gpu_draft(ds, cfg, I)
    compared, excused = compare_draft(o, g, "c5-full")
    print(f"c5 draft: compared {compared}, excused {excused}")


def test_c5_cycle_full(ora, ds, c5):
    """One cycle of the production loop on the RNN head: the confidences of the cycle two
    before (drafted on the GPU, checked against the oracle) give the batch capacity, this
    cycle's confidences rank the candidates (two-step-lag schedule), and verification takes
    this cycle's drafted block with its float bias rows."""
    cfg, I, _ = c5
    g = _gpu_draft(ds, cfg, I)
    g_lag = _gpu_draft(ds, cfg, I, cycle=CYCLE - 2)
    print("c5 cycle: oracle RNN draft of the lagged cycle", flush=True)
    o_lag = _oracle_draft(ora, cfg, I, cycle=CYCLE - 2)
    compare_draft(o_lag, g_lag, "c5-lag-full")
    ell = _schedule_both(ora, ds, cfg, g["c"], ora.ASYNC_LAG2,
                         c_lag=np.asarray(g_lag["c"], np.float32))
    print(f"c5 cycle: lagged schedule admits {int(ell.sum())} of {cfg.R * cfg.gamma}")
    assert ell.sum() > 0
    target = _target(cfg, I, g["bias_rows"])
    _verify_both(ora, ds, cfg, I, target, g["x"], g["lse"], g["logit_x"],
                 np.asarray(g["bias_rows"], np.float32), ell, "c5-full")


def test_c3_parallel_drafter_full(ora, ds):
    """The draft without the sequential head at the headline sizes (what the head's cost
    is measured against): the oracle's Markov draft with W2 = 0."""
    cfg = synth.CONFIGS["c3"]
    I = synth.inputs(cfg)
    print("c3 parallel drafter: oracle with W2 = 0", flush=True)
    o = ora.draft_markov(I["U"], I["h"], I["W1"], np.zeros_like(I["W2"]), I["w"], I["x0"], 0,
                         CYCLE)
    g = ds.draft_parallel(T(I["U"]), T(I["h"]), T(I["W1"]), T(I["w"]), T(I["x0"]), 0, CYCLE)
    g = {k: N(v) for k, v in g.items()}
    g["bias_rows"] = synth.bf16_to_f32(g["bias_rows"])
    compared, excused = compare_draft(o, g, "c3-parallel-full")
    print(f"c3 parallel drafter: compared {compared}, excused {excused}")
