"""Helpers shared by the GPU parity tests: device transfer, oracle runs on the same seeded
inputs, and the agreement rules (tokens identical except counted near-ties, probabilities
within 1e-4 absolute).

Every token or acceptance decision a parity test compares is counted in TALLY, and every
mismatch the near-tie rule excuses is counted too.  The rate over the whole session must
stay below 0.1 % (asserted by tests/test_zy_parity_tally.py, which runs after the parity
tests, and printed in the terminal summary by conftest.py)."""
import numpy as np

TOL_P = 1e-4       # probabilities, confidences, c*
TIE_GAP = 1e-3     # a token may differ only where the oracle's top-two Gumbel scores are closer
ACC_EXCUSE = 1e-4  # an acceptance test may differ only where |u - p/q| is below this
EXCUSE_RATE = 1e-3  # excused / compared over the session

TALLY = {"compared": 0, "excused": 0, "cases": []}


def record(label, compared, excused):
    """Add one parity case's counts to the session tally."""
    TALLY["compared"] += int(compared)
    TALLY["excused"] += int(excused)
    TALLY["cases"].append((label, int(compared), int(excused)))


def dev():
    import torch
    return torch.device("cuda:0")


def T(a):
    """numpy -> device tensor (uint16 arrays are bf16 bit patterns); device tensors pass."""
    import torch
    if isinstance(a, torch.Tensor):
        return a
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev())


def W2T(W2):
    """The pages' W2 [r][V] (numpy) on the device, re-laid out to W2t [V][r] by the
    library's dspark_w2_relayout (the layout the hot-path calls take)."""
    import draft_sampling_scheduling_amd as ds
    return ds.w2_relayout(T(W2))


def N(t):
    import torch
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def compare_draft(o, g, label=""):
    """Token-by-token agreement of a drafted block.  Per request, positions are compared up
    to the first token mismatch (later positions are conditioned on different prefixes); a
    mismatch must sit on an oracle near-tie.  Returns (compared, excused)."""
    xg, xo = g["x"], o["x"]
    R, gamma = xo.shape
    compared = excused = 0
    for q in range(R):
        for k in range(gamma):
            compared += 1
            # outputs of step k depend on x_{k-1}, which matched
            assert abs(g["c"][q, k] - o["c"][q, k]) <= TOL_P, (label, q, k, g["c"][q, k], o["c"][q, k])
            assert abs(g["lse"][q, k] - o["lse"][q, k]) <= TOL_P, (label, q, k, g["lse"][q, k], o["lse"][q, k])
            if "z" in g and "z" in o:  # confidence logit before the temperature
                assert abs(g["z"][q, k] - o["z"][q, k]) <= TOL_P * (1 + abs(o["z"][q, k])), (
                    label, q, k, g["z"][q, k], o["z"][q, k])
            if xg[q, k] != xo[q, k]:
                near = min(o["gap_blk"][q, k], o["gap_in"][q, k]) < TIE_GAP
                assert near, (label, "token mismatch off a near-tie", q, k, xg[q, k], xo[q, k],
                              o["gap_blk"][q, k], o["gap_in"][q, k])
                excused += 1
                break
            qg = np.exp(np.float64(g["logit_x"][q, k]) - np.float64(g["lse"][q, k]))
            qo = np.exp(o["logit_x"][q, k] - o["lse"][q, k])
            assert abs(qg - qo) <= TOL_P, (label, q, k, qg, qo)
            np.testing.assert_allclose(np.asarray(g["bias_rows"][q, k], np.float64),
                                       o["bias_rows"][q, k], atol=1e-4 if g["bias_rows"].dtype == np.float32 else 0)
    record(label, compared, excused)
    return compared, excused


def compare_verify(o, g, ell, label):
    """Agreement of a verification: c* within 1e-4 on every verified row (NaN after),
    accepted counts and emitted tokens identical.  An accepted count may differ only where
    the first differing acceptance test is a near-tie (|u - p/q| below ACC_EXCUSE, oracle
    values); the final token (correction or bonus) only at a sampler near-tie.  Counts
    sum(ell) + R decisions.  Returns the number excused."""
    excused = 0
    R = len(ell)
    if "x_next" in g:  # the next cycle's anchors: the last emitted token of every request
        assert np.array_equal(g["x_next"], g["y"][np.arange(R), g["n_acc"]]), label
    for q in range(R):
        L = ell[q]
        np.testing.assert_allclose(g["c_star"][q, :L], o["c_star"][q, :L], atol=TOL_P, err_msg=label)
        assert np.all(np.isnan(g["c_star"][q, L:])), (label, q)
        if g["n_acc"][q] != o["n_acc"][q]:
            j = min(g["n_acc"][q], o["n_acc"][q])  # first differing acceptance test (0-based)
            gap = abs(o["u_acc"][q, j] - o["pq_ratio"][q, j])
            assert gap < ACC_EXCUSE, (label, "acceptance differs off a near-tie", q, j, gap)
            excused += 1
            continue
        na = o["n_acc"][q]
        assert np.array_equal(g["y"][q, :na], o["y"][q, :na]), (label, q)
        assert np.all(g["y"][q, na + 1:] == -1), (label, q)
        if g["y"][q, na] != o["y"][q, na]:
            assert min(o["gap_blk"][q], o["gap_in"][q]) < TIE_GAP, (label, "final token differs", q)
            excused += 1
    record(label, int(np.sum(ell)) + R, excused)
    return excused
