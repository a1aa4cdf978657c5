"""SPS(B) profiling with the verification pass as the stand-in engine (digest page,
Module E): the profiled steps/s are positive, fall as the batch grows, and the interpolated
table drives the scheduler.  A measurement has no oracle: these are its properties."""
import numpy as np
import pytest

from draft_sampling_scheduling_amd import synth
from tests.gpu_util import N, T

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ds():
    import draft_sampling_scheduling_amd as ds
    ds.lib()
    return ds


def test_profile_and_schedule(ds):
    cfg = synth.scaled(synth.CONFIGS["c2"], R=64, gamma=4, V=16384, d=256)
    I = synth.inputs(cfg)
    W2t = np.ascontiguousarray(I["W2"].T)
    d = ds.draft_markov(T(I["U"]), T(I["h"]), T(I["W1"]), T(W2t), T(I["w"]), T(I["x0"]), 0, 1)
    noise, fresh = synth.target_parts(cfg, range(cfg.R), 1)
    U = synth.decode(cfg, I["U"])
    br = synth.bf16_to_f32(N(d["bias_rows"]))
    logits = U + np.matmul(br, synth.decode(cfg, I["W2"]))
    target = synth.encode(cfg, np.concatenate([logits, fresh[:, None, :]], axis=1) + noise)
    R, G = cfg.R, cfg.gamma
    B_list = [R, R + 64, R + 128, R + 192, R * (1 + G)]
    sps = ds.sps_profile(T(target), T(I["U"]), T(W2t), d["bias_rows"], d["x"], d["lse"],
                         d["logit_x"], B_list, reps=5)
    print("SPS(B) at", B_list, ":", sps)
    assert np.all(np.isfinite(sps)) and np.all(sps > 0)
    assert sps[0] > 1.1 * sps[-1]  # verifying R*gamma more rows costs time
    table = ds.sps_interpolate(B_list, sps, R, R * (1 + G))
    assert table.shape == (R * G + 1,) and np.all(table > 0)
    s = ds.schedule(d["c"], T(table), R, ds.GLOBAL)
    ell = N(s["ell"])
    assert np.all((ell >= 0) & (ell <= G))
    stats = N(s["stats"])
    assert stats[0] == R + ell.sum()
