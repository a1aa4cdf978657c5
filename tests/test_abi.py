"""Host-side checks of the C ABI: the library builds, loads and exports every declared
symbol, and rejects bad arguments before touching a device (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def ds():
    import draft_sampling_scheduling_amd as ds
    if not os.path.exists(ds.LIB_PATH):
        from draft_sampling_scheduling_amd import build
        build.build()
    ds.lib()
    return ds


def _declared():
    src = open(os.path.join(ROOT, "include", "dspark.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(ds):
    names = _declared()
    assert len(names) == 23, names
    for n in names:
        assert hasattr(ds.lib(), n), n
    assert set(names) == set(ds.EXPORTS)
    assert "gfx950" in ds.version()


def test_workspace_sizes(ds):
    a = ds.draft_workspace_bytes(256, 8, 151936, 256, 4096)
    b = ds.draft_rnn_workspace_bytes(256, 8, 151936, 256, 4096)
    assert 0 < a < b
    assert ds.verify_workspace_bytes(256, 8, 151936, 256) > 0
    assert ds.draft_workspace_bytes(4, 4, 1001, 16, 64) == 0   # V % 8 != 0
    assert ds.draft_workspace_bytes(4, 4, 1024, 48, 64) == 0   # r not a power of two
    assert ds.draft_workspace_bytes(4, 0, 1024, 16, 64) == 0   # gamma < 1


FAKE = C.c_void_p(0x1000)  # never dereferenced: these calls return before any launch


def test_draft_rejects_bad_arguments(ds):
    L = ds.lib()
    ws = ds.draft_workspace_bytes(4, 4, 1024, 16, 64)

    def call(R=4, gamma=4, V=1024, r=16, d=64, dt=ds.F32, U=FAKE, ws_bytes=ws, cycle=0):
        return L.dspark_draft_markov(R, gamma, V, r, d, dt, U, FAKE, FAKE, FAKE, FAKE, None,
                                     FAKE, 0, cycle, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                     FAKE, ws_bytes, None)

    assert call(V=1001) == ds.EINVAL
    assert call(r=24) == ds.EINVAL
    assert call(dt=7) == ds.EINVAL
    assert call(U=None) == ds.EINVAL
    assert call(ws_bytes=ws - 1) == ds.EWORKSPACE
    assert call(cycle=1 << 28) == ds.EINVAL
    assert call(R=0) == ds.OK  # empty batch: nothing to do


def test_draft_noalloc_rejects_before_launch(ds):
    L = ds.lib()
    assert ds.draft_markov_noalloc_max_bytes() == 16 << 20

    def call(R=4, gamma=4, V=1024, r=16, d=64):
        return L.dspark_draft_markov_noalloc(R, gamma, V, r, d, ds.BF16, FAKE, FAKE, FAKE, FAKE,
                                             FAKE, None, FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE,
                                             FAKE, FAKE, None, None)

    assert call(V=1001) == ds.EINVAL
    assert call(r=24) == ds.EINVAL
    # the shapes need more than the library's scratch array
    assert ds.draft_workspace_bytes(1100, 8, 151936, 256, 4096) > 16 << 20
    assert call(R=1100, gamma=8, V=151936, r=256, d=4096) == ds.ERANGE
    assert ds.draft_workspace_bytes(512, 16, 151936, 256, 5120) <= 16 << 20
    assert call(R=0) == ds.OK


def test_w2_relayout_rejects_bad_arguments(ds):
    L = ds.lib()
    other = C.c_void_p(0x2000)
    assert L.dspark_w2_relayout(1001, 16, ds.BF16, FAKE, other, None) == ds.EINVAL
    assert L.dspark_w2_relayout(1024, 48, ds.BF16, FAKE, other, None) == ds.EINVAL
    assert L.dspark_w2_relayout(1024, 16, 5, FAKE, other, None) == ds.EINVAL
    assert L.dspark_w2_relayout(1024, 16, ds.F32, None, other, None) == ds.EINVAL
    assert L.dspark_w2_relayout(1024, 16, ds.F32, FAKE, FAKE, None) == ds.EINVAL  # aliased


def test_read_probe_arguments(ds):
    """The read probe's argument checks return before anything reaches the device."""
    L = ds.lib()
    sink = C.c_void_p(0x2000)
    ev = C.c_void_p(0x3000)
    assert L.dspark_read_probe(None, 1024, 4, sink, None, None, None) == ds.EINVAL
    assert L.dspark_read_probe(FAKE, 1024, 4, None, None, None, None) == ds.EINVAL
    assert L.dspark_read_probe(FAKE, 1000, 4, sink, None, None, None) == ds.EINVAL  # 16-byte whole
    assert L.dspark_read_probe(C.c_void_p(0x1008), 1024, 4, sink, None, None, None) == ds.EINVAL
    assert L.dspark_read_probe(FAKE, 1024, 0, sink, None, None, None) == ds.EINVAL
    assert L.dspark_read_probe(FAKE, 1024, 65537, sink, None, None, None) == ds.EINVAL
    assert L.dspark_read_probe(FAKE, 1024, 4, sink, None, ev, None) == ds.EINVAL    # one event


def test_schedule_rejects_bad_arguments(ds):
    L = ds.lib()

    def call(R=4, gamma=3, sps_B0=4, sps_len=13, mode=ds.SYNC_BREAK, c_lag=None, R_lag=0):
        return L.dspark_schedule(R, gamma, FAKE, c_lag, R_lag, FAKE, sps_B0, sps_len, mode,
                                 FAKE, None, None, None, None, 0, None)

    assert call(sps_len=12) == ds.ERANGE      # must reach R(1+gamma) = 16
    assert call(sps_B0=5, sps_len=20) == ds.ERANGE
    assert call(mode=5) == ds.EINVAL
    assert call(mode=ds.ASYNC_LAG2) == ds.EINVAL  # no lagged confidences
    assert call(mode=ds.ASYNC_LAG2, c_lag=FAKE, R_lag=8) == ds.ERANGE  # 8*(1+3) > 16
    assert call(R=1024, gamma=9, sps_B0=1, sps_len=20000) == ds.EINVAL  # R*gamma > 8192
    assert call(gamma=0) == ds.EINVAL
    assert call() == ds.EWORKSPACE  # no workspace
    ws = ds.schedule_workspace_bytes(4, 3)
    assert ws >= 4 * 3 * 12
    assert ds.schedule_workspace_bytes(1024, 9) == 0  # R*gamma > 8192
    assert L.dspark_schedule(4, 3, FAKE, None, 0, FAKE, 4, 13, ds.SYNC_BREAK, FAKE, None, None,
                             None, FAKE, ws - 1, None) == ds.EWORKSPACE


def test_verify_rejects_bad_arguments(ds):
    L = ds.lib()
    ws = ds.verify_workspace_bytes(4, 4, 1024, 16)

    def call(dt=ds.BF16, bdt=ds.BF16, ws_bytes=ws, V=1024):
        return L.dspark_verify(4, 4, V, 16, dt, FAKE, FAKE, FAKE, FAKE, bdt, FAKE, FAKE, FAKE,
                               FAKE, 0, 0, FAKE, FAKE, FAKE, None, None, FAKE, ws_bytes, None)

    assert call(dt=ds.F32, bdt=ds.BF16) == ds.EINVAL  # bias rows must be float or dt
    assert call(ws_bytes=ws - 1) == ds.EWORKSPACE
    assert call(V=1020) == ds.EINVAL


def test_sts_rejects_bad_arguments(ds):
    import numpy as np
    L = ds.lib()
    assert ds.sts_workspace_bytes(0, 10, 15) == 0
    assert ds.sts_workspace_bytes(1000, 129, 1) == 0       # G > 128
    assert ds.sts_workspace_bytes(1000, 64, 65) == 0       # G * nbins > 4096
    assert ds.sts_workspace_bytes((1 << 24) + 1, 4, 4) == 0
    ws = ds.sts_workspace_bytes(1000, 3, 10)
    assert ws >= 1000 * 8

    def call(grid=(0.5, 1.0, 2.0), N=1000, gamma=4, nbins=10, ws_bytes=ws):
        g = np.asarray(grid, np.float32)
        return L.dspark_sts_fit(N, gamma, FAKE, FAKE, g.ctypes.data_as(C.c_void_p), len(g),
                                nbins, FAKE, None, FAKE, ws_bytes, None)

    assert call(grid=(0.5, 0.0, 2.0)) == ds.EINVAL
    assert call(grid=(0.5, -1.0)) == ds.EINVAL
    assert call(grid=(0.5, float("nan"))) == ds.EINVAL
    assert call(grid=(0.5, float("inf"))) == ds.EINVAL
    assert call(gamma=0) == ds.EINVAL
    assert call(gamma=65) == ds.EINVAL
    assert call(ws_bytes=ws - 1) == ds.EWORKSPACE


def test_train_forward_rejects_bad_arguments(ds):
    L = ds.lib()
    ws = ds.train_forward_workspace_bytes(4, 4, 1024, 16, 64)
    assert ws > 0
    assert ds.train_forward_workspace_bytes(4, 4, 1001, 16, 64) == 0
    assert ds.train_forward_workspace_bytes(2048, 8, 151936, 256, 4096) == 0  # >= 4 GiB rows

    def call(dt=ds.BF16, V=1024, r=16, ws_bytes=ws, R=4):
        return L.dspark_train_forward(R, 4, V, r, 64, dt, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, 0.1, 0.9, 1.0, None, None, None, None, None,
                                      None, FAKE, ws_bytes, None)

    assert call(dt=ds.F32) == ds.EINVAL
    assert call(V=1020) == ds.EINVAL
    assert call(r=24) == ds.EINVAL
    assert call(ws_bytes=ws - 1) == ds.EWORKSPACE
    assert call(R=0) == ds.OK


def test_decode_rejects_bad_arguments(ds):
    L = ds.lib()
    ws = ds.decode_workspace_bytes(4, 4, 1024, 16, 8, ds.BF16)
    assert ws > 0
    assert ds.decode_workspace_bytes(4, 4, 1020, 16, 8, ds.BF16) == 0
    assert ds.decode_workspace_bytes(0, 4, 1024, 16, 8, ds.BF16) == 0

    def call(policy=3, sps=None, sps_B0=1, sps_len=0, ws_bytes=ws, ncycles=2, dt=ds.BF16):
        return L.dspark_decode_run(4, 4, 1024, 16, 8, dt, ncycles, FAKE, FAKE, FAKE, FAKE,
                                   FAKE, None, FAKE, FAKE, policy, 0.0, sps, sps_B0, sps_len,
                                   0, FAKE, FAKE, FAKE, None, FAKE, ws_bytes, None)

    assert call(policy=5) == ds.EINVAL
    assert call(policy=0) == ds.EINVAL                          # no SPS table
    assert call(policy=0, sps=FAKE, sps_len=10) == ds.ERANGE    # must reach R(1+gamma) = 20
    assert call(ws_bytes=ws - 1) == ds.EWORKSPACE
    assert call(ncycles=-1) == ds.EINVAL
    assert call(dt=7) == ds.EINVAL


def test_sps_interpolate(ds):
    import numpy as np
    out = ds.sps_interpolate([10, 14, 20], [4.0, 2.0, 1.0], 10, 20)
    expect = [4.0, 3.5, 3.0, 2.5, 2.0, 2 - 1 / 6, 2 - 2 / 6, 1.5, 2 - 4 / 6, 2 - 5 / 6, 1.0]
    np.testing.assert_allclose(out, expect, rtol=1e-6)
    assert ds.sps_interpolate([5], [3.0], 5, 5).tolist() == [3.0]
    np.testing.assert_allclose(ds.sps_interpolate([0, 8], [1.0, 9.0], 3, 5), [4.0, 5.0, 6.0])
    for bad in (([10, 10], [1.0, 1.0]), ([10, 12], [1.0, 0.0])):
        with pytest.raises(ds.DsparkError):
            ds.sps_interpolate(*bad, 10, 10)
    with pytest.raises(ds.DsparkError):
        ds.sps_interpolate([10, 20], [2.0, 1.0], 9, 15)


def test_sps_profile_rejects_bad_arguments(ds):
    import numpy as np
    L = ds.lib()

    def call(B, R=4, gamma=2):
        bl = np.asarray(B, np.int32)
        out = np.zeros(len(B), np.float32)
        return L.dspark_sps_profile(R, gamma, 1024, 16, ds.BF16, FAKE, FAKE, FAKE, FAKE,
                                    ds.BF16, FAKE, FAKE, FAKE, len(B),
                                    bl.ctypes.data_as(C.c_void_p), 3,
                                    out.ctypes.data_as(C.c_void_p), FAKE, FAKE, FAKE, FAKE,
                                    None, FAKE, 1 << 20, None)

    assert call([3, 8]) == ds.ERANGE       # below R
    assert call([4, 13]) == ds.ERANGE      # above R(1+gamma) = 12
    assert call([8, 6]) == ds.EINVAL       # not ascending
