"""dspark_w2_relayout (W2 [r][V] as the pages write it -> W2t [V][r]) against the numpy
transpose: bit-exact for bf16 and float, ragged vocabularies (not a multiple of the 64-id
tile) and every supported rank, and the full vocabulary of the headline workload."""
import numpy as np
import pytest

from tests.gpu_util import N, T

pytestmark = pytest.mark.gpu

CASES = [(1000, 16, "bf16"), (1000, 32, "f32"), (4104, 64, "bf16"), (640, 128, "f32"),
         (32000, 256, "bf16"), (151936, 256, "bf16"), (8, 16, "f32")]


@pytest.mark.parametrize("V,r,dt", CASES, ids=[f"V{c[0]}-r{c[1]}-{c[2]}" for c in CASES])
def test_relayout_is_the_transpose(V, r, dt):
    import draft_sampling_scheduling_amd as ds
    rng = np.random.default_rng(V + r)
    W2 = rng.standard_normal((r, V), dtype=np.float32)
    if dt == "bf16":
        W2 = W2.view(np.uint32).__rshift__(16).astype(np.uint16)  # any bit patterns will do
    out = N(ds.w2_relayout(T(W2)))
    assert out.dtype == W2.dtype and out.shape == (V, r)
    assert np.array_equal(out, np.ascontiguousarray(W2.T))
