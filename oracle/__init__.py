"""Python access to the plain CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg
may import this package; the HIP library and its binding never do.  It shares no code with
the GPU path.  Arrays are numpy; bf16 operands are passed as their uint16 bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1
SYNC_BREAK, GLOBAL, ASYNC_LAG2 = 0, 1, 2
S_DRAFT_BLK, S_DRAFT_IN, S_ACCEPT, S_RESID_BLK, S_RESID_IN, S_BONUS_BLK, S_BONUS_IN = range(7)
VB = 64


def build() -> str:
    """Compile liboracle.so with gcc (fp64, IEEE, OpenMP over requests)."""
    subprocess.check_call(
        ["gcc", "-O2", "-std=c99", "-Wall", "-fopenmp", "-fPIC", "-shared", "oracle.c",
         "-o", "liboracle.so", "-lm"], cwd=_HERE)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(_LIB_PATH)
        vp, i32p, f32p, f64p, i64p = (C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_float),
                                      C.POINTER(C.c_double), C.POINTER(C.c_int64))
        u32p = C.POINTER(C.c_uint32)
        L.ora_philox4x32_10.argtypes = [u32p, u32p, u32p]
        L.ora_rand_word.argtypes = [C.c_uint64, C.c_uint64, C.c_int, C.c_uint32, C.c_uint32,
                                    C.c_uint32]
        L.ora_rand_word.restype = C.c_uint32
        for f in (L.ora_uniform, L.ora_gumbel):
            f.argtypes = L.ora_rand_word.argtypes
            f.restype = C.c_double
        L.ora_sample_two_level.argtypes = [C.c_int, f64p, C.c_uint64, C.c_uint64, C.c_int,
                                           C.c_int, C.c_uint32, C.c_uint32, f64p, f64p]
        L.ora_sample_two_level.restype = C.c_int
        L.ora_sample_trials.argtypes = [C.c_int, f64p, C.c_uint64, C.c_uint64, C.c_int,
                                        C.c_int, C.c_long, i64p]
        common = [C.c_int] * 6 + [vp, vp, vp, vp]
        outs = [i32p, f64p, f64p, f64p, f64p, f64p, f64p, f64p]
        L.ora_draft_markov.argtypes = common + [f32p, f32p, i32p, i32p, C.c_uint64,
                                                C.c_uint64] + outs
        L.ora_draft_rnn.argtypes = common + [vp, f32p, f32p, i32p, i32p, C.c_uint64,
                                             C.c_uint64] + outs
        L.ora_draft_markov.restype = L.ora_draft_rnn.restype = C.c_int
        L.ora_schedule.argtypes = [C.c_int, C.c_int, f32p, f32p, C.c_int, f32p, C.c_int,
                                   C.c_int, C.c_int, i32p, f32p, f64p, f64p]
        L.ora_schedule.restype = C.c_int
        L.ora_schedule_literal.argtypes = [C.c_int, C.c_int, f32p, f32p, C.c_int, C.c_int,
                                           C.c_int, i32p, f64p]
        L.ora_schedule_literal.restype = C.c_int
        L.ora_verify.argtypes = ([C.c_int] * 5 + [vp, vp, vp, f64p, i32p, i32p, i32p, C.c_uint64,
                                 C.c_uint64, i32p, i32p, f64p, f64p, f64p, f64p, f64p])
        L.ora_verify.restype = C.c_int
        L.ora_sts_fit.argtypes = [C.c_int, C.c_int, f32p, i32p, f32p, C.c_int, C.c_int, f32p,
                                  f64p]
        L.ora_sts_fit.restype = C.c_int
        L.ora_train_forward.argtypes = ([C.c_int] * 6 + [vp, vp, vp, vp, f32p, vp, i32p, i32p,
                                        f64p, f64p, f64p, f64p, f64p, f64p])
        L.ora_train_forward.restype = C.c_int
        L.ora_decode_run.argtypes = ([C.c_int] * 7 + [vp, vp, vp, vp, f32p, f32p, vp, i32p,
                                     C.c_int, C.c_float, f32p, C.c_int, C.c_int, C.c_uint64,
                                     i32p, i32p, i64p])
        L.ora_decode_run.restype = C.c_int
        L.ora_num_threads.restype = C.c_int
        L.ora_set_num_threads.argtypes = [C.c_int]
        L.ora_set_num_threads.restype = None
        _lib = L
    return _lib


def _p(a, ct):
    return None if a is None else a.ctypes.data_as(C.POINTER(ct))


def _vp(a):
    return None if a is None else C.c_void_p(a.ctypes.data)


def _dt_of(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"operand dtype must be uint16 (bf16 bits) or float32, got {a.dtype}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return lib().ora_num_threads()


def set_num_threads(n: int) -> None:
    lib().ora_set_num_threads(int(n))


def philox(ctr, key) -> np.ndarray:
    c = _c(ctr, np.uint32)
    k = _c(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().ora_philox4x32_10(_p(c, C.c_uint32), _p(k, C.c_uint32), _p(out, C.c_uint32))
    return out


def rand_word(seed, cycle, stream, r, k, i) -> int:
    return int(lib().ora_rand_word(seed, cycle, stream, r, k, i))


def uniform(seed, cycle, stream, r, k, i) -> float:
    return float(lib().ora_uniform(seed, cycle, stream, r, k, i))


def gumbel(seed, cycle, stream, r, k, i) -> float:
    return float(lib().ora_gumbel(seed, cycle, stream, r, k, i))


def sample_two_level(l, seed, cycle, stream_blk, stream_in, r, k):
    l = _c(l, np.float64)
    gb, gi = C.c_double(), C.c_double()
    x = lib().ora_sample_two_level(l.size, _p(l, C.c_double), seed, cycle, stream_blk,
                                   stream_in, r, k, C.byref(gb), C.byref(gi))
    return x, gb.value, gi.value


def sample_trials(l, seed, cycle, stream_blk, stream_in, ntrials) -> np.ndarray:
    l = _c(l, np.float64)
    counts = np.zeros(l.size, np.int64)
    lib().ora_sample_trials(l.size, _p(l, C.c_double), seed, cycle, stream_blk, stream_in,
                            ntrials, _p(counts, C.c_int64))
    return counts


def _draft(U, h, W1, W2, w, x0, seed, cycle, W_gco=None, req_ids=None, temps=None):
    U, h, W1, W2 = (np.ascontiguousarray(a) for a in (U, h, W1, W2))
    dt = _dt_of(U)
    for a in (h, W1, W2) + ((W_gco,) if W_gco is not None else ()):
        if _dt_of(a) != dt:
            raise TypeError("all big operands must share one dtype")
    R, gamma, V = U.shape
    rank = W1.shape[1]
    d = h.shape[2]
    assert W1.shape == (V, rank) and W2.shape == (rank, V) and h.shape[:2] == (R, gamma)
    w = _c(w, np.float32)
    assert w.shape == (d + rank,)
    x0 = _c(x0, np.int32)
    rid = None if req_ids is None else _c(req_ids, np.int32)
    assert rid is None or rid.shape == (R,)
    tp = None if temps is None else _c(temps, np.float32)
    assert tp is None or tp.shape == (gamma,)
    x = np.zeros((R, gamma), np.int32)
    c, zc, lse, logit_x, gb, gi = (np.zeros((R, gamma)) for _ in range(6))
    bias_rows = np.zeros((R, gamma, rank))
    args = [R, gamma, V, rank, d, dt, _vp(U), _vp(h), _vp(W1), _vp(W2)]
    tail = [_p(w, C.c_float), _p(tp, C.c_float), _p(x0, C.c_int32), _p(rid, C.c_int32), seed,
            cycle, _p(x, C.c_int32), _p(c, C.c_double), _p(zc, C.c_double),
            _p(lse, C.c_double), _p(logit_x, C.c_double),
            _p(bias_rows, C.c_double), _p(gb, C.c_double), _p(gi, C.c_double)]
    if W_gco is None:
        rc = lib().ora_draft_markov(*args, *tail)
    else:
        W_gco = np.ascontiguousarray(W_gco)
        assert W_gco.shape == (3 * rank, 2 * rank + d)
        rc = lib().ora_draft_rnn(*args, _vp(W_gco), *tail)
    if rc != 0:
        raise ValueError(f"oracle draft rejected its arguments (rc={rc})")
    return dict(x=x, c=c, z=zc, lse=lse, logit_x=logit_x, bias_rows=bias_rows, gap_blk=gb,
                gap_in=gi)


def draft_markov(U, h, W1, W2, w, x0, seed=0, cycle=0, req_ids=None, temps=None):
    """Markov-head draft (eqs. 4, 5, 7).  W2 is [rank][V] as on the pages.  temps: the
    STS temperatures per position (Module D), None = 1."""
    return _draft(U, h, W1, W2, w, x0, seed, cycle, req_ids=req_ids, temps=temps)


def draft_rnn(U, h, W1, W2, W_gco, w, x0, seed=0, cycle=0, req_ids=None, temps=None):
    """RNN-head draft (eq. 6, confidence eq. 7)."""
    return _draft(U, h, W1, W2, w, x0, seed, cycle, W_gco=W_gco, req_ids=req_ids, temps=temps)


def sts_fit(z, n_acc, grid, nbins=15):
    """STS calibration (Module D): per-position temperatures from held-out confidence
    logits z [N][gamma] and accepted lengths n_acc [N].  Returns (T [gamma], ece [gamma])."""
    z = _c(z, np.float32)
    N, gamma = z.shape
    n_acc = _c(n_acc, np.int32)
    grid = _c(grid, np.float32)
    assert n_acc.shape == (N,)
    T = np.zeros(gamma, np.float32)
    ece = np.zeros(gamma)
    rc = lib().ora_sts_fit(N, gamma, _p(z, C.c_float), _p(n_acc, C.c_int32),
                           _p(grid, C.c_float), grid.size, nbins, _p(T, C.c_float),
                           _p(ece, C.c_double))
    if rc != 0:
        raise ValueError(f"oracle sts_fit rejected its arguments (rc={rc})")
    return T, ece



ALPHA = (0.1, 0.9, 1.0)  # (a_ce, a_tv, a_conf), Module F eq. (12) defaults


def train_forward(U, h, W1, W2, w, target, x0, xstar, alpha=ALPHA):
    """Training objective forward (Module F, eqs. 8-12) on teacher-forced blocks with the
    Markov head.  target [R][gamma][V]; xstar [R][gamma] reference tokens (x*_0 = x0).
    Returns dict(c_star, c, logq, tv [R][gamma]; loss [R][4] = L_ce, L_tv, L_conf, L)."""
    U, h, W1, W2, target = (np.ascontiguousarray(a) for a in (U, h, W1, W2, target))
    dt = _dt_of(U)
    for a in (h, W1, W2, target):
        if _dt_of(a) != dt:
            raise TypeError("all big operands must share one dtype")
    R, gamma, V = U.shape
    rank = W1.shape[1]
    d = h.shape[2]
    assert W1.shape == (V, rank) and W2.shape == (rank, V) and h.shape[:2] == (R, gamma)
    assert target.shape == (R, gamma, V)
    w = _c(w, np.float32)
    assert w.shape == (d + rank,)
    x0 = _c(x0, np.int32)
    xs = _c(xstar, np.int32)
    assert x0.shape == (R,) and xs.shape == (R, gamma)
    al = _c(alpha, np.float64)
    assert al.shape == (3,)
    cs, c, lq, tv = (np.zeros((R, gamma)) for _ in range(4))
    loss = np.zeros((R, 4))
    rc = lib().ora_train_forward(R, gamma, V, rank, d, dt, _vp(U), _vp(h), _vp(W1), _vp(W2),
                                 _p(w, C.c_float), _vp(target), _p(x0, C.c_int32),
                                 _p(xs, C.c_int32), _p(al, C.c_double), _p(cs, C.c_double),
                                 _p(c, C.c_double), _p(lq, C.c_double), _p(tv, C.c_double),
                                 _p(loss, C.c_double))
    if rc != 0:
        raise ValueError(f"oracle train_forward rejected its arguments (rc={rc})")
    return dict(c_star=cs, c=c, logq=lq, tv=tv, loss=loss)



FIXED, THRESHOLD = 3, 4  # length policies of the driver beyond the scheduler's modes


def decode_run(Ub, Hb, W1, W2, w, Tb, x0, ncycles, policy=SYNC_BREAK, threshold=0.0,
               sps=None, sps_B0=1, seed=0, temps=None):
    """Multi-cycle decode on a toy chain (bigram target Tb [V][V], table backbone Ub
    [V][gamma][V], Hb [V][gamma][d]).  Returns dict(tokens [R][ncycles*(gamma+1)],
    n_emitted [R], tested [gamma], accepted [gamma], sum_ell, emitted, request_cycles)."""
    Ub, Hb, W1, W2, Tb = (np.ascontiguousarray(a) for a in (Ub, Hb, W1, W2, Tb))
    dt = _dt_of(Ub)
    for a in (Hb, W1, W2, Tb):
        if _dt_of(a) != dt:
            raise TypeError("all big operands must share one dtype")
    V, gamma, _ = Ub.shape
    rank = W1.shape[1]
    d = Hb.shape[2]
    assert Ub.shape == (V, gamma, V) and Hb.shape[:2] == (V, gamma) and Tb.shape == (V, V)
    assert W1.shape == (V, rank) and W2.shape == (rank, V)
    w = _c(w, np.float32)
    x0 = _c(x0, np.int32)
    R = x0.shape[0]
    sp = None if sps is None else _c(sps, np.float32)
    tp = None if temps is None else _c(temps, np.float32)
    tokens = np.zeros((R, ncycles * (gamma + 1)), np.int32)
    n_em = np.zeros(R, np.int32)
    st = np.zeros(2 * gamma + 3, np.int64)
    rc = lib().ora_decode_run(R, gamma, V, rank, d, dt, ncycles, _vp(Ub), _vp(Hb), _vp(W1),
                              _vp(W2), _p(w, C.c_float), _p(tp, C.c_float), _vp(Tb),
                              _p(x0, C.c_int32), policy, threshold, _p(sp, C.c_float), sps_B0,
                              0 if sp is None else sp.size, seed, _p(tokens, C.c_int32),
                              _p(n_em, C.c_int32), _p(st, C.c_int64))
    if rc != 0:
        raise ValueError(f"oracle decode_run rejected its arguments (rc={rc})")
    return dict(tokens=tokens, n_emitted=n_em, tested=st[:gamma], accepted=st[gamma:2 * gamma],
                sum_ell=int(st[2 * gamma]), emitted=int(st[2 * gamma + 1]),
                request_cycles=int(st[2 * gamma + 2]))


def schedule(c, sps, sps_B0, mode=SYNC_BREAK, c_lag=None, trace=False):
    """Prefix scheduler.  Returns dict(ell, a, stats=(B, tau, Theta, n_adm), theta)."""
    c = _c(c, np.float32)
    R, gamma = c.shape
    sps = _c(sps, np.float32)
    cl = None if c_lag is None else _c(c_lag, np.float32)
    R_lag = 0 if cl is None else cl.shape[0]
    ell = np.zeros(R, np.int32)
    a = np.zeros((R, gamma), np.float32)
    stats = np.zeros(4)
    theta = np.zeros(R * gamma + 1) if trace else None
    rc = lib().ora_schedule(R, gamma, _p(c, C.c_float), _p(cl, C.c_float), R_lag,
                            _p(sps, C.c_float), sps_B0, sps.size, mode, _p(ell, C.c_int32),
                            _p(a, C.c_float), _p(stats, C.c_double), _p(theta, C.c_double))
    if rc != 0:
        raise ValueError(f"oracle schedule rejected its arguments (rc={rc})")
    return dict(ell=ell, a=a, stats=stats, theta=theta)


def schedule_literal(c, sps, sps_B0, brk=True):
    """Algorithm 1 with single-precision running sums (the literal reading).  Returns
    dict(ell, theta) with theta the float Theta of every prefix (NaN past |E|)."""
    c = _c(c, np.float32)
    R, gamma = c.shape
    sps = _c(sps, np.float32)
    ell = np.zeros(R, np.int32)
    theta = np.zeros(R * gamma + 1)
    rc = lib().ora_schedule_literal(R, gamma, _p(c, C.c_float), _p(sps, C.c_float), sps_B0,
                                    sps.size, 1 if brk else 0, _p(ell, C.c_int32),
                                    _p(theta, C.c_double))
    if rc != 0:
        raise ValueError(f"oracle schedule_literal rejected its arguments (rc={rc})")
    return dict(ell=ell, theta=theta)


def schedule_rc(c, sps, sps_B0, mode=SYNC_BREAK, c_lag=None) -> int:
    """Return code only (error-path tests)."""
    c = _c(c, np.float32)
    R, gamma = c.shape
    sps = _c(sps, np.float32)
    cl = None if c_lag is None else _c(c_lag, np.float32)
    ell = np.zeros(R, np.int32)
    return lib().ora_schedule(R, gamma, _p(c, C.c_float), _p(cl, C.c_float),
                              0 if cl is None else cl.shape[0], _p(sps, C.c_float), sps_B0,
                              sps.size, mode, _p(ell, C.c_int32), None, None, None)


def verify(target, U, W2, bias_rows, x, ell, seed=0, cycle=0, req_ids=None):
    """Rejection-sampling verification (returns dict of n_acc, y, c_star, ...)."""
    target, U, W2 = (np.ascontiguousarray(a) for a in (target, U, W2))
    dt = _dt_of(U)
    if _dt_of(target) != dt or _dt_of(W2) != dt:
        raise TypeError("target, U and W2 must share one dtype")
    R, gamma, V = U.shape
    rank = W2.shape[0]
    assert target.shape == (R, gamma + 1, V) and W2.shape == (rank, V)
    bias_rows = _c(bias_rows, np.float64)
    assert bias_rows.shape == (R, gamma, rank)
    x = _c(x, np.int32)
    ell = _c(ell, np.int32)
    rid = None if req_ids is None else _c(req_ids, np.int32)
    n_acc = np.zeros(R, np.int32)
    y = np.zeros((R, gamma + 1), np.int32)
    c_star, pq, ua = (np.zeros((R, gamma)) for _ in range(3))
    gb, gi = np.zeros(R), np.zeros(R)
    rc = lib().ora_verify(R, gamma, V, rank, dt, _vp(target), _vp(U), _vp(W2),
                          _p(bias_rows, C.c_double), _p(x, C.c_int32), _p(ell, C.c_int32),
                          _p(rid, C.c_int32), seed, cycle, _p(n_acc, C.c_int32), _p(y, C.c_int32),
                          _p(c_star, C.c_double), _p(pq, C.c_double), _p(ua, C.c_double),
                          _p(gb, C.c_double), _p(gi, C.c_double))
    if rc != 0:
        raise ValueError(f"oracle verify rejected its arguments (rc={rc})")
    return dict(n_acc=n_acc, y=y, c_star=c_star, pq_ratio=pq, u_acc=ua, gap_blk=gb,
                gap_in=gi)
