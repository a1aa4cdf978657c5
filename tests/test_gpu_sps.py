"""SPS(B) profiling with the verification pass as the stand-in engine (digest page,
Module E): the profiled steps/s are positive, fall as the batch grows, and the interpolated
table drives the scheduler.  A measurement has no oracle: these are its properties."""
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


def test_profile_and_schedule(ds):
    cfg = synth.scaled(synth.CONFIGS["c2"], R=64, gamma=4, V=16384, d=256)
    I = synth.inputs(cfg)
    W2t = W2T(I["W2"])
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


def test_profiled_batches_spread_the_lengths(ds):
    """Each profiled batch B is made of R requests and B - R verified rows spread as evenly
    as possible, earlier requests first: ell[q] = floor((B-R)/R) + (q < (B-R) mod R), so
    R + sum(ell) = B (the batch the timing stands for)."""
    import torch
    cfg = synth.scaled(synth.CONFIGS["c2"], R=37, gamma=5, V=4096, d=128)
    I = synth.inputs(cfg)
    W2t = W2T(I["W2"])
    d = ds.draft_markov(T(I["U"]), T(I["h"]), T(I["W1"]), W2t, T(I["w"]), T(I["x0"]), 0, 2)
    noise, fresh = synth.target_parts(cfg, range(cfg.R), 2)
    U = synth.decode(cfg, I["U"])
    br = synth.bf16_to_f32(N(d["bias_rows"]))
    logits = U + np.matmul(br, synth.decode(cfg, I["W2"]))
    target = T(synth.encode(cfg, np.concatenate([logits, fresh[:, None, :]], axis=1) + noise))
    R, G = cfg.R, cfg.gamma
    ell = torch.empty(R, dtype=torch.int32, device="cuda:0")
    for B in (R, R + 1, R + 17, R + R, 2 * R + 5, R * (1 + G) - 1, R * (1 + G)):
        sps = ds.sps_profile(target, T(I["U"]), W2t, d["bias_rows"], d["x"], d["lse"],
                             d["logit_x"], [B], reps=1, ell=ell)
        e = N(ell)
        q = np.arange(R)
        want = (B - R) // R + (q < (B - R) % R)
        assert np.array_equal(e, want.astype(np.int32)), (B, e)
        assert R + int(e.sum()) == B
        assert np.all(np.isfinite(sps)) and sps[0] > 0
