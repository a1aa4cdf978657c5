"""Helpers shared by the GPU parity tests: device transfer, oracle runs on the same seeded
inputs, and the agreement rules (tokens identical except counted near-ties, probabilities
within 1e-4 absolute)."""
import numpy as np

TOL_P = 1e-4       # probabilities, confidences, c*
TIE_GAP = 1e-3     # a token may differ only where the oracle's top-two Gumbel scores are closer
ACC_EXCUSE = 1e-4  # an acceptance test may differ only where |u - p/q| is below this


def dev():
    import torch
    return torch.device("cuda:0")


def T(a):
    """numpy -> device tensor (uint16 arrays are bf16 bit patterns)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev())


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
    return compared, excused


def excuse_budget(compared):
    return 1 + int(0.001 * compared)
