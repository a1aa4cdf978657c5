"""GPU verification (dspark_verify) against the oracle on inputs the oracle drafted:
accepted counts and emitted tokens identical except counted near-ties, c* within 1e-4."""
import numpy as np
import pytest

from draft_sampling_scheduling_amd import synth
from tests.gpu_util import N, T, compare_verify, W2T

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ds():
    import draft_sampling_scheduling_amd as ds
    ds.lib()
    return ds


def _inputs(ora, cfg, cycle, ell_kind, rnn=False, edit_target=None):
    I = synth.inputs(cfg)
    if rnn:
        d = ora.draft_rnn(I["U"], I["h"], I["W1"], I["W2"], I["W_gco"], I["w"], I["x0"], 0, cycle)
    else:
        d = ora.draft_markov(I["U"], I["h"], I["W1"], I["W2"], I["w"], I["x0"], 0, cycle)
    # synthetic target-model stand-in: the drafted logits plus noise; bonus row fresh
    U = synth.decode(cfg, I["U"]).astype(np.float64)
    W2 = synth.decode(cfg, I["W2"]).astype(np.float64)
    logits = U + np.einsum("qkr,rv->qkv", d["bias_rows"], W2)
    noise, fresh = synth.target_parts(cfg, range(cfg.R), cycle)
    tgt = np.concatenate([logits, fresh[:, None, :]], axis=1) + noise
    if edit_target is not None:
        edit_target(tgt)
    target = synth.encode(cfg, tgt.astype(np.float32))
    rng = np.random.default_rng(cycle)
    if ell_kind == "sched":
        s = ora.schedule(d["c"].astype(np.float32), synth.sps_table(cfg), cfg.sps_B0, 0)
        ell = s["ell"]
    elif ell_kind == "full":
        ell = np.full(cfg.R, cfg.gamma, np.int32)
    elif ell_kind == "zero":  # nothing verified: every request draws from its row 1
        ell = np.zeros(cfg.R, np.int32)
    else:
        ell = rng.integers(0, cfg.gamma + 1, cfg.R).astype(np.int32)
        ell[0] = 0
        ell[-1] = cfg.gamma
    return I, d, target, ell


CASES = [
    ("c1-sched", "c1", {}, "sched"),
    ("c1-random", "c1", dict(R=9, V=1000), "random"),
    ("c2-random", "c2", dict(R=48, gamma=5, V=6000, d=256), "random"),
    ("c2-full", "c2", dict(R=33, gamma=4, V=4096, d=128, r=128), "full"),
    ("c2-zero", "c2", dict(R=21, gamma=4, V=3000, d=128), "zero"),
    ("c2-sched", "c2", dict(R=64, gamma=4, V=8192, d=256), "sched"),
    ("c3-law", "c3", dict(R=40, gamma=6, V=16384, d=256), "random"),
]


@pytest.mark.parametrize("name,base,kw,ell_kind", CASES, ids=[c[0] for c in CASES])
def test_verify_parity(ora, ds, name, base, kw, ell_kind):
    cfg = synth.scaled(synth.CONFIGS[base], **kw)
    cycle = 4
    I, d, target, ell = _inputs(ora, cfg, cycle, ell_kind)
    o = ora.verify(target, I["U"], I["W2"], d["bias_rows"], d["x"], ell, seed=0, cycle=cycle)
    brows = synth.encode(cfg, d["bias_rows"].astype(np.float32))  # exact: rows of W1
    W2t = W2T(I["W2"])
    g = ds.verify(T(target), T(I["U"]), T(W2t), T(brows), T(d["x"]),
                  T(d["lse"].astype(np.float32)), T(d["logit_x"].astype(np.float32)), T(ell),
                  seed=0, cycle=cycle)
    g = {k: N(v) for k, v in g.items()}
    excused = compare_verify(o, g, ell, name)
    print(f"{name}: rows {int(ell.sum())}, accepted {int(o['n_acc'].sum())}, excused {excused}")


def test_verify_rnn_float_bias_rows(ora, ds):
    cfg = synth.scaled(synth.CONFIGS["c5"], R=24, gamma=4, V=4096, r=64, d=128)
    cycle = 2
    I, d, target, ell = _inputs(ora, cfg, cycle, "random", rnn=True)
    o = ora.verify(target, I["U"], I["W2"], d["bias_rows"], d["x"], ell, seed=0, cycle=cycle)
    W2t = W2T(I["W2"])
    g = ds.verify(T(target), T(I["U"]), T(W2t), T(d["bias_rows"].astype(np.float32)), T(d["x"]),
                  T(d["lse"].astype(np.float32)), T(d["logit_x"].astype(np.float32)), T(ell),
                  seed=0, cycle=cycle)
    g = {k: N(v) for k, v in g.items()}
    excused = compare_verify(o, g, ell, "rnn")


def _spikes(tgt):
    """Single logits far above the rest of their row, placed where the target normaliser's
    first estimate of a window's largest logit (each lane's first chunk: the window's first
    512 ids) cannot see them: 100 above the row (its sums would leave the float range, so
    that window is redone against its exact maximum), 60 above (kept: large but finite
    sums), in the last, partial window, and on bonus rows."""
    R, G1, V = tgt.shape
    top = float(tgt.max())
    for q in range(R):
        for j in range(G1):
            if q % 3 == 0:
                tgt[q, j, 1000 + 37 * j] = top + 100.0
            elif q % 3 == 1:
                tgt[q, j, V - 5] = top + 60.0
            elif j == G1 - 1:
                tgt[q, j, 4096 + 600 + q] = top + 100.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_verify_logit_spikes(ora, ds, dtype):
    base = dict(R=12, gamma=4, V=6000, d=128)
    cfg = synth.scaled(synth.CONFIGS["c2" if dtype == "bf16" else "c1"], **base)
    cycle = 6
    I, d, target, ell = _inputs(ora, cfg, cycle, "random", edit_target=_spikes)
    o = ora.verify(target, I["U"], I["W2"], d["bias_rows"], d["x"], ell, seed=0, cycle=cycle)
    brows = synth.encode(cfg, d["bias_rows"].astype(np.float32))
    W2t = W2T(I["W2"])
    g = ds.verify(T(target), T(I["U"]), T(W2t), T(brows), T(d["x"]),
                  T(d["lse"].astype(np.float32)), T(d["logit_x"].astype(np.float32)), T(ell),
                  seed=0, cycle=cycle)
    g = {k: N(v) for k, v in g.items()}
    compare_verify(o, g, ell, f"spikes-{dtype}")


def test_length_fault_bit(ora, ds):
    import torch
    cfg = synth.scaled(synth.CONFIGS["c2"], R=4, gamma=3, V=1024, d=64)
    I, d, target, ell = _inputs(ora, cfg, 0, "random")
    ell = ell.copy()
    ell[1] = 9
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    W2t = W2T(I["W2"])
    brows = synth.encode(cfg, d["bias_rows"].astype(np.float32))
    ds.verify(T(target), T(I["U"]), T(W2t), T(brows), T(d["x"]), T(d["lse"].astype(np.float32)),
              T(d["logit_x"].astype(np.float32)), T(ell), status=status)
    assert int(N(status)[0]) & ds.FAULT_LEN


def test_verify_deterministic(ora, ds):
    """Three verifications of the same drafted block (same seed and cycle) give
    bit-identical accepted counts, tokens and c*."""
    cfg = synth.scaled(synth.CONFIGS["c3"], R=40, gamma=6, V=16384, d=256)
    I, d, target, ell = _inputs(ora, cfg, 5, "random")
    W2t = W2T(I["W2"])
    brows = synth.encode(cfg, d["bias_rows"].astype(np.float32))
    runs = []
    for _ in range(3):
        g = ds.verify(T(target), T(I["U"]), W2t, T(brows), T(d["x"]),
                      T(d["lse"].astype(np.float32)), T(d["logit_x"].astype(np.float32)),
                      T(ell), seed=0, cycle=5)
        runs.append({k: N(v).tobytes() for k, v in g.items()})
    assert runs[0] == runs[1] == runs[2]
