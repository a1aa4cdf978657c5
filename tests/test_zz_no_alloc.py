"""The allocation-free draft entry point (dspark_draft_markov_noalloc) against the
workspace one (dspark_draft_markov): identical outputs on two calls in a row, the second
with a smaller batch and vocabulary, so the shared scratch array holds the first call's
contents when the second starts."""
import numpy as np
import pytest

from draft_sampling_scheduling_amd import synth
from tests.gpu_util import N, T

pytestmark = pytest.mark.gpu


def _operands(cfg):
    I = synth.inputs(cfg)
    W2t = np.ascontiguousarray(I["W2"].T)
    return [T(I["U"]), T(I["h"]), T(I["W1"]), T(W2t), T(I["w"]), T(I["x0"])]


def test_noalloc_matches_workspace_entry_point():
    import torch

    import draft_sampling_scheduling_amd as ds
    ds.lib()
    big = synth.scaled(synth.CONFIGS["c3"], R=200, gamma=6, V=40000, d=512)
    small = synth.scaled(synth.CONFIGS["c2"], R=37, gamma=3, V=6016, d=128, r=64)
    for name, cfg in (("big", big), ("small", small)):
        print(f"no-alloc draft, {name}: R={cfg.R} gamma={cfg.gamma} V={cfg.V} r={cfg.r}",
              flush=True)
        ops = _operands(cfg)
        st_a = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        st_b = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        a = ds.draft_markov_noalloc(*ops, seed=7, cycle=5, status=st_a)
        b = ds.draft_markov(*ops, seed=7, cycle=5, status=st_b)
        a = {k: N(v) for k, v in a.items()}
        b = {k: N(v) for k, v in b.items()}
        assert int(N(st_a)[0]) == 0 and int(N(st_b)[0]) == 0
        for k in ("x", "c", "z", "lse", "logit_x", "bias_rows"):
            assert np.array_equal(a[k], b[k]), (name, k)
