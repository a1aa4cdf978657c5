"""DSpark draft -> schedule -> verify hot path on MI355X: Python binding of libdspark.so.

Thin ctypes layer over the C ABI in include/dspark.h: it checks shapes and dtypes,
allocates outputs and workspaces with PyTorch (device memory only) and passes raw device
pointers plus torch's current HIP stream.  Every step of the path runs in the library's
HIP kernels; there is no fallback: if the library is missing the calls raise.

Operand dtypes: torch.bfloat16 or torch.float32 for U, h, W1, W2t, W_gco and the target
logits (all of one call share one dtype); float32 for w and the confidences; int32 tokens.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdspark.so")

F32, BF16 = 0, 1
SYNC_BREAK, GLOBAL, ASYNC_LAG2 = 0, 1, 2
FIXED, THRESHOLD = 3, 4  # decode-driver length policies beyond the scheduler's modes
OK, EINVAL, ERANGE, EWORKSPACE, EDEVICE = 0, -1, -2, -3, -4
FAULT_TOKEN, FAULT_CONF, FAULT_LEN = 1, 2, 4
EXPORTS = ("dspark_draft_workspace_bytes", "dspark_draft_markov", "dspark_draft_markov_timed",
           "dspark_draft_markov_noalloc_max_bytes", "dspark_draft_markov_noalloc",
           "dspark_draft_parallel",
           "dspark_draft_rnn_workspace_bytes", "dspark_draft_rnn",
           "dspark_schedule_workspace_bytes", "dspark_schedule",
           "dspark_verify_workspace_bytes", "dspark_verify",
           "dspark_sts_workspace_bytes", "dspark_sts_fit",
           "dspark_train_forward_workspace_bytes", "dspark_train_forward",
           "dspark_decode_workspace_bytes", "dspark_decode_run",
           "dspark_sps_profile", "dspark_sps_interpolate", "dspark_w2_relayout",
           "dspark_read_probe", "dspark_version")

_lib = None


class DsparkError(RuntimeError):
    def __init__(self, fn: str, rc: int):
        names = {EINVAL: "EINVAL", ERANGE: "ERANGE", EWORKSPACE: "EWORKSPACE",
                 EDEVICE: "EDEVICE"}
        super().__init__(f"{fn} returned {names.get(rc, rc)}")
        self.rc = rc


def lib():
    """Load libdspark.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python __graft_entry__.py` "
                               "(or draft_sampling_scheduling_amd.build.build())")
        # load PyTorch's HIP runtime first: the library then binds to that same runtime
        # (one libamdhip64.so.7 per process), so torch streams are valid handles for it
        import torch  # noqa: F401

        L = C.CDLL(LIB_PATH)
        i, u64, sz, vp = C.c_int, C.c_uint64, C.c_size_t, C.c_void_p
        L.dspark_draft_workspace_bytes.argtypes = [i] * 5
        L.dspark_draft_workspace_bytes.restype = sz
        L.dspark_draft_rnn_workspace_bytes.argtypes = [i] * 5
        L.dspark_draft_rnn_workspace_bytes.restype = sz
        L.dspark_draft_markov.argtypes = ([i] * 6 + [vp] * 7 + [u64, u64] + [vp] * 7 +
                                          [vp, sz, vp])
        L.dspark_draft_markov.restype = i
        L.dspark_draft_markov_timed.argtypes = L.dspark_draft_markov.argtypes + [vp, vp]
        L.dspark_draft_markov_timed.restype = i
        L.dspark_draft_markov_noalloc_max_bytes.argtypes = []
        L.dspark_draft_markov_noalloc_max_bytes.restype = sz
        L.dspark_draft_markov_noalloc.argtypes = [i] * 6 + [vp] * 7 + [u64, u64] + [vp] * 8
        L.dspark_draft_markov_noalloc.restype = i
        L.dspark_draft_parallel.argtypes = ([i] * 6 + [vp] * 6 + [u64, u64] + [vp] * 7 +
                                            [vp, sz, vp])
        L.dspark_draft_parallel.restype = i
        L.dspark_draft_rnn.argtypes = ([i] * 6 + [vp] * 8 + [u64, u64] + [vp] * 7 +
                                       [vp, sz, vp])
        L.dspark_draft_rnn.restype = i
        L.dspark_schedule_workspace_bytes.argtypes = [i, i]
        L.dspark_schedule_workspace_bytes.restype = sz
        L.dspark_schedule.argtypes = [i, i, vp, vp, i, vp, i, i, i, vp, vp, vp, vp, vp, sz, vp]
        L.dspark_schedule.restype = i
        L.dspark_verify_workspace_bytes.argtypes = [i] * 4
        L.dspark_verify_workspace_bytes.restype = sz
        L.dspark_verify.argtypes = ([i] * 5 + [vp] * 4 + [i] + [vp] * 4 + [u64, u64] +
                                    [vp] * 5 + [vp, sz, vp])
        L.dspark_verify.restype = i
        L.dspark_sts_workspace_bytes.argtypes = [i] * 3
        L.dspark_sts_workspace_bytes.restype = sz
        L.dspark_sts_fit.argtypes = [i, i, vp, vp, vp, i, i, vp, vp, vp, sz, vp]
        L.dspark_sts_fit.restype = i
        L.dspark_train_forward_workspace_bytes.argtypes = [i] * 5
        L.dspark_train_forward_workspace_bytes.restype = sz
        f = C.c_float
        L.dspark_train_forward.argtypes = ([i] * 6 + [vp] * 8 + [f, f, f] + [vp] * 6 +
                                           [vp, sz, vp])
        L.dspark_train_forward.restype = i
        L.dspark_decode_workspace_bytes.argtypes = [i] * 6
        L.dspark_decode_workspace_bytes.restype = sz
        L.dspark_decode_run.argtypes = ([i] * 7 + [vp] * 8 + [i, f, vp, i, i, u64] + [vp] * 4 +
                                        [vp, sz, vp])
        L.dspark_decode_run.restype = i
        L.dspark_sps_profile.argtypes = ([i] * 5 + [vp] * 4 + [i] + [vp] * 3 + [i, vp, i] +
                                         [vp] * 6 + [vp, sz, vp])
        L.dspark_sps_profile.restype = i
        L.dspark_sps_interpolate.argtypes = [i, vp, vp, i, i, vp]
        L.dspark_sps_interpolate.restype = i
        L.dspark_w2_relayout.argtypes = [i, i, i, vp, vp, vp]
        L.dspark_w2_relayout.restype = i
        L.dspark_read_probe.argtypes = [vp, sz, i, vp, vp, vp, vp]
        L.dspark_read_probe.restype = i
        L.dspark_version.restype = C.c_char_p
        _lib = L
    return _lib


def version() -> str:
    return lib().dspark_version().decode()


# ----------------------------------------------------------------------------------------
# torch plumbing
# ----------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"operand dtype must be bfloat16 or float32, got {t.dtype}")


def _chk(t, name, shape=None, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _ws(nbytes: int, device, ws=None):
    torch = _torch()
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError("workspace too small")
        return ws
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def _raise(fn, rc):
    if rc != OK:
        raise DsparkError(fn, rc)


# ----------------------------------------------------------------------------------------
# entry points (same names as the C ABI without the prefix)
# ----------------------------------------------------------------------------------------
def w2_relayout(W2, *, out=None):
    """W2 [r][V] (the pages' layout) -> W2t [V][r], the layout the draft, verify, training
    and decode calls take (dspark_w2_relayout; device tensors, same dtype)."""
    torch = _torch()
    _chk(W2, "W2")
    r, V = W2.shape
    dt = _dt(W2)
    if out is None:
        out = torch.empty((V, r), dtype=W2.dtype, device=W2.device)
    _chk(out, "W2t", (V, r), W2.dtype)
    _raise("dspark_w2_relayout", lib().dspark_w2_relayout(V, r, dt, _p(W2), _p(out), _stream()))
    return out


def read_probe(buf, grid=2048, *, sink=None, events=None):
    """Benchmark hook: a plain streaming read of the device tensor `buf` (its bytes, a
    multiple of 16) by `grid` workgroups; returns the [grid] int32 sink, whose XOR is the
    XOR of buf's 32-bit words (dspark_read_probe).  events=(begin, end): raw hipEvent_t
    handles the dispatch timestamps."""
    torch = _torch()
    _chk(buf, "buf")
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(grid, dtype=torch.int32, device=buf.device)
    _chk(sink, "sink", (grid,), torch.int32)
    ev0, ev1 = events if events is not None else (None, None)
    _raise("dspark_read_probe",
           lib().dspark_read_probe(_p(buf), nbytes, grid, _p(sink), _stream(), ev0, ev1))
    return sink


def draft_workspace_bytes(R, gamma, V, r, d) -> int:
    return int(lib().dspark_draft_workspace_bytes(R, gamma, V, r, d))


def draft_rnn_workspace_bytes(R, gamma, V, r, d) -> int:
    return int(lib().dspark_draft_rnn_workspace_bytes(R, gamma, V, r, d))


def _draft(rnn, U, h, W1, W2t, w, x0, seed, cycle, W_gco=None, temps=None, out=None, ws=None,
           status=None, events=None, parallel=False):
    torch = _torch()
    _chk(U, "U")
    R, gamma, V = U.shape
    dt = _dt(U)
    r = W1.shape[1]
    d = h.shape[2]
    _chk(h, "h", (R, gamma, d), U.dtype)
    _chk(W1, "W1", (V, r), U.dtype)
    if not parallel:
        _chk(W2t, "W2t", (V, r), U.dtype)
    _chk(w, "w", (d + r,), torch.float32)
    _chk(x0, "x0", (R,), torch.int32)
    if temps is not None:
        _chk(temps, "temps", (gamma,), torch.float32)
    if rnn:
        _chk(W_gco, "W_gco", (3 * r, 2 * r + d), U.dtype)
    dev = U.device
    if out is None:
        out = dict(
            x=torch.empty((R, gamma), dtype=torch.int32, device=dev),
            c=torch.empty((R, gamma), dtype=torch.float32, device=dev),
            z=torch.empty((R, gamma), dtype=torch.float32, device=dev),
            lse=torch.empty((R, gamma), dtype=torch.float32, device=dev),
            logit_x=torch.empty((R, gamma), dtype=torch.float32, device=dev),
            bias_rows=torch.empty((R, gamma, r), dtype=torch.float32 if rnn else U.dtype,
                                  device=dev))
    nbytes = (draft_rnn_workspace_bytes if rnn else draft_workspace_bytes)(R, gamma, V, r, d)
    if nbytes == 0 and R > 0:
        raise DsparkError("dspark_draft_workspace_bytes", EINVAL)
    ws = _ws(nbytes, dev, ws)
    args = [R, gamma, V, r, d, dt, _p(U), _p(h), _p(W1)]
    if not parallel:
        args.append(_p(W2t))
    if rnn:
        args.append(_p(W_gco))
    args += [_p(w), _p(temps), _p(x0), seed, cycle, _p(out["x"]), _p(out["c"]),
             _p(out.get("z")), _p(out["lse"]), _p(out["logit_x"]), _p(out["bias_rows"]), _p(status), _p(ws),
             ws.numel() * ws.element_size(), _stream()]
    fn = "dspark_draft_rnn" if rnn else ("dspark_draft_parallel" if parallel else
                                         "dspark_draft_markov")
    if events is not None:  # (begin, end): ctypes arrays of gamma hipEvent_t each
        if parallel:
            raise ValueError("the timed hook is the Markov head's")
        fn = "dspark_draft_markov_timed"
        args += [C.cast(events[0], C.c_void_p), C.cast(events[1], C.c_void_p)]
    _raise(fn, getattr(lib(), fn)(*args))
    return out


def draft_markov(U, h, W1, W2t, w, x0, seed=0, cycle=0, *, temps=None, out=None, ws=None,
                 status=None, events=None):
    """Markov-head draft; returns dict(x, c, z, lse, logit_x, bias_rows) (device tensors).
    temps: [gamma] float32 STS temperatures (None: 1).  A caller-supplied `out` without a
    "z" entry skips that output.  events=(begin, end) arrays of gamma hipEvent_t selects
    the timed variant."""
    return _draft(False, U, h, W1, W2t, w, x0, seed, cycle, temps=temps, out=out, ws=ws,
                  status=status, events=events)


def draft_parallel(U, h, W1, w, x0, seed=0, cycle=0, *, temps=None, out=None, ws=None,
                   status=None):
    """The parallel block's drafter without the sequential head: x_k from softmax(U_k);
    same outputs as draft_markov (bf16 operands)."""
    return _draft(False, U, h, W1, None, w, x0, seed, cycle, temps=temps, out=out, ws=ws,
                  status=status, parallel=True)


def draft_markov_noalloc(U, h, W1, W2t, w, x0, seed=0, cycle=0, *, temps=None, out=None,
                         status=None):
    """dspark_draft_markov_noalloc: the Markov-head draft with the library's own device
    workspace (no workspace argument; calls that overlap on one GPU race).  Same results
    as draft_markov."""
    torch = _torch()
    _chk(U, "U")
    R, gamma, V = U.shape
    dt = _dt(U)
    r = W1.shape[1]
    d = h.shape[2]
    _chk(h, "h", (R, gamma, d), U.dtype)
    _chk(W1, "W1", (V, r), U.dtype)
    _chk(W2t, "W2t", (V, r), U.dtype)
    _chk(w, "w", (d + r,), torch.float32)
    _chk(x0, "x0", (R,), torch.int32)
    if temps is not None:
        _chk(temps, "temps", (gamma,), torch.float32)
    dev = U.device
    if out is None:
        out = dict(
            x=torch.empty((R, gamma), dtype=torch.int32, device=dev),
            c=torch.empty((R, gamma), dtype=torch.float32, device=dev),
            z=torch.empty((R, gamma), dtype=torch.float32, device=dev),
            lse=torch.empty((R, gamma), dtype=torch.float32, device=dev),
            logit_x=torch.empty((R, gamma), dtype=torch.float32, device=dev),
            bias_rows=torch.empty((R, gamma, r), dtype=U.dtype, device=dev))
    rc = lib().dspark_draft_markov_noalloc(
        R, gamma, V, r, d, dt, _p(U), _p(h), _p(W1), _p(W2t), _p(w), _p(temps), _p(x0), seed,
        cycle, _p(out["x"]), _p(out["c"]), _p(out.get("z")), _p(out["lse"]),
        _p(out["logit_x"]), _p(out["bias_rows"]), _p(status), _stream())
    _raise("dspark_draft_markov_noalloc", rc)
    return out


def draft_markov_noalloc_max_bytes() -> int:
    return int(lib().dspark_draft_markov_noalloc_max_bytes())


def draft_rnn(U, h, W1, W2t, W_gco, w, x0, seed=0, cycle=0, *, temps=None, out=None, ws=None,
              status=None):
    """RNN-head draft; bias_rows is float32."""
    return _draft(True, U, h, W1, W2t, w, x0, seed, cycle, W_gco=W_gco, temps=temps, out=out,
                  ws=ws, status=status)


def schedule_workspace_bytes(R, gamma) -> int:
    return int(lib().dspark_schedule_workspace_bytes(R, gamma))


def schedule(c, sps, sps_B0, mode=SYNC_BREAK, c_lag=None, *, out=None, ws=None, status=None):
    """Prefix scheduler; returns dict(ell, a, stats) (device tensors)."""
    torch = _torch()
    _chk(c, "c", dtype=torch.float32)
    R, gamma = c.shape
    _chk(sps, "sps", dtype=torch.float32)
    R_lag = 0
    if c_lag is not None:
        _chk(c_lag, "c_lag", dtype=torch.float32)
        R_lag = c_lag.shape[0]
    dev = c.device
    if out is None:
        out = dict(ell=torch.empty(R, dtype=torch.int32, device=dev),
                   a=torch.empty((R, gamma), dtype=torch.float32, device=dev),
                   stats=torch.empty(4, dtype=torch.float64, device=dev))
    ws = _ws(schedule_workspace_bytes(R, gamma), dev, ws)
    rc = lib().dspark_schedule(R, gamma, _p(c), _p(c_lag), R_lag, _p(sps), sps_B0,
                               sps.numel(), mode, _p(out["ell"]), _p(out["a"]),
                               _p(out["stats"]), _p(status), _p(ws),
                               ws.numel() * ws.element_size(), _stream())
    _raise("dspark_schedule", rc)
    return out


def verify_workspace_bytes(R, gamma, V, r) -> int:
    return int(lib().dspark_verify_workspace_bytes(R, gamma, V, r))


def verify(target, U, W2t, bias_rows, x, lse, logit_x, ell, seed=0, cycle=0, *, out=None,
           ws=None, status=None):
    """Verification; returns dict(n_acc, y, c_star, x_next) (device tensors).  x_next [R]
    holds y[q][n_acc[q]], the next cycle's anchors; a caller's `out` may map it to the tensor
    the next draft call takes as x0 (or leave it out: then it is not written)."""
    torch = _torch()
    _chk(U, "U")
    R, gamma, V = U.shape
    dt = _dt(U)
    r = W2t.shape[1]
    _chk(target, "target", (R, gamma + 1, V), U.dtype)
    _chk(W2t, "W2t", (V, r), U.dtype)
    _chk(bias_rows, "bias_rows", (R, gamma, r))
    bdt = _dt(bias_rows)
    _chk(x, "x", (R, gamma), torch.int32)
    _chk(lse, "lse", (R, gamma), torch.float32)
    _chk(logit_x, "logit_x", (R, gamma), torch.float32)
    _chk(ell, "ell", (R,), torch.int32)
    dev = U.device
    if out is None:
        out = dict(n_acc=torch.empty(R, dtype=torch.int32, device=dev),
                   y=torch.empty((R, gamma + 1), dtype=torch.int32, device=dev),
                   c_star=torch.empty((R, gamma), dtype=torch.float32, device=dev),
                   x_next=torch.empty(R, dtype=torch.int32, device=dev))
    x_next = out.get("x_next")
    if x_next is not None:
        _chk(x_next, "x_next", (R,), torch.int32)
    nbytes = verify_workspace_bytes(R, gamma, V, r)
    if nbytes == 0 and R > 0:
        raise DsparkError("dspark_verify_workspace_bytes", EINVAL)
    ws = _ws(nbytes, dev, ws)
    rc = lib().dspark_verify(R, gamma, V, r, dt, _p(target), _p(U), _p(W2t), _p(bias_rows),
                             bdt, _p(x), _p(lse), _p(logit_x), _p(ell), seed, cycle,
                             _p(out["n_acc"]), _p(out["y"]), _p(out["c_star"]), _p(x_next),
                             _p(status),
                             _p(ws), ws.numel() * ws.element_size(), _stream())
    _raise("dspark_verify", rc)
    return out


def sts_workspace_bytes(N, G, nbins) -> int:
    return int(lib().dspark_sts_workspace_bytes(N, G, nbins))


def sts_fit(z, n_acc, grid, nbins=15, *, out=None, ws=None):
    """STS temperatures, fitted left to right on held-out (z, accepted length) samples.
    z [N][gamma] float32 and n_acc [N] int32 are device tensors; grid is a host sequence of
    candidate temperatures.  Returns dict(T [gamma] float32, ece [gamma] float64)."""
    import numpy as np
    torch = _torch()
    _chk(z, "z", dtype=torch.float32)
    if z.dim() != 2:
        raise ValueError("z must be [N][gamma]")
    N, gamma = z.shape
    _chk(n_acc, "n_acc", (N,), torch.int32)
    g = np.ascontiguousarray(np.asarray(grid, dtype=np.float32).ravel())
    dev = z.device
    if out is None:
        out = dict(T=torch.empty(gamma, dtype=torch.float32, device=dev),
                   ece=torch.empty(gamma, dtype=torch.float64, device=dev))
    nbytes = sts_workspace_bytes(N, len(g), nbins)
    if nbytes == 0:
        raise DsparkError("dspark_sts_workspace_bytes", EINVAL)
    ws = _ws(nbytes, dev, ws)
    rc = lib().dspark_sts_fit(N, gamma, _p(z), _p(n_acc),
                              g.ctypes.data_as(C.c_void_p), len(g), nbins, _p(out["T"]),
                              _p(out.get("ece")), _p(ws), ws.numel() * ws.element_size(),
                              _stream())
    _raise("dspark_sts_fit", rc)
    return out


ALPHA = (0.1, 0.9, 1.0)  # (a_ce, a_tv, a_conf): the loss mix of the training objective


def train_forward_workspace_bytes(R, gamma, V, r, d) -> int:
    return int(lib().dspark_train_forward_workspace_bytes(R, gamma, V, r, d))


def train_forward(U, h, W1, W2t, w, target, x0, xstar, alpha=ALPHA, *, out=None, ws=None,
                  status=None):
    """Training-objective forward on teacher-forced blocks (Markov head, bf16 operands).
    Returns dict(c_star, c, logq, tv [R][gamma]; loss [R][4] = L_ce, L_tv, L_conf, L)."""
    torch = _torch()
    _chk(U, "U")
    R, gamma, V = U.shape
    dt = _dt(U)
    r = W1.shape[1]
    d = h.shape[2]
    _chk(h, "h", (R, gamma, d), U.dtype)
    _chk(W1, "W1", (V, r), U.dtype)
    _chk(W2t, "W2t", (V, r), U.dtype)
    _chk(w, "w", (d + r,), torch.float32)
    _chk(target, "target", (R, gamma, V), U.dtype)
    _chk(x0, "x0", (R,), torch.int32)
    _chk(xstar, "xstar", (R, gamma), torch.int32)
    dev = U.device
    if out is None:
        out = {k: torch.empty((R, gamma), dtype=torch.float32, device=dev)
               for k in ("c_star", "c", "logq", "tv")}
        out["loss"] = torch.empty((R, 4), dtype=torch.float32, device=dev)
    nbytes = train_forward_workspace_bytes(R, gamma, V, r, d)
    if nbytes == 0:
        raise DsparkError("dspark_train_forward_workspace_bytes", EINVAL)
    ws = _ws(nbytes, dev, ws)
    a = [float(x) for x in alpha]
    rc = lib().dspark_train_forward(R, gamma, V, r, d, dt, _p(U), _p(h), _p(W1), _p(W2t),
                                    _p(w), _p(target), _p(x0), _p(xstar), a[0], a[1], a[2],
                                    _p(out.get("c_star")), _p(out.get("c")),
                                    _p(out.get("logq")), _p(out.get("tv")),
                                    _p(out.get("loss")), _p(status), _p(ws),
                                    ws.numel() * ws.element_size(), _stream())
    _raise("dspark_train_forward", rc)
    return out


def decode_workspace_bytes(R, gamma, V, r, d, dt) -> int:
    return int(lib().dspark_decode_workspace_bytes(R, gamma, V, r, d, dt))


def decode_run(Ub, Hb, W1, W2t, w, Tb, x0, ncycles, policy=SYNC_BREAK, threshold=0.0,
               sps=None, sps_B0=1, seed=0, temps=None, *, out=None, ws=None, status=None):
    """Multi-cycle decode on a toy chain: bigram target Tb [V][V], table backbone Ub
    [V][gamma][V] and Hb [V][gamma][d] (device tensors).  Returns dict(tokens
    [R][ncycles*(gamma+1)], n_emitted [R], stats [2*gamma+3] int64)."""
    torch = _torch()
    _chk(Ub, "Ub")
    V, gamma, _ = Ub.shape
    dt = _dt(Ub)
    r = W1.shape[1]
    d = Hb.shape[2]
    _chk(Ub, "Ub", (V, gamma, V))
    _chk(Hb, "Hb", (V, gamma, d), Ub.dtype)
    _chk(W1, "W1", (V, r), Ub.dtype)
    _chk(W2t, "W2t", (V, r), Ub.dtype)
    _chk(w, "w", (d + r,), torch.float32)
    _chk(Tb, "Tb", (V, V), Ub.dtype)
    _chk(x0, "x0", dtype=torch.int32)
    R = x0.shape[0]
    if temps is not None:
        _chk(temps, "temps", (gamma,), torch.float32)
    if sps is not None:
        _chk(sps, "sps", dtype=torch.float32)
    dev = Ub.device
    if out is None:
        out = dict(tokens=torch.empty((R, ncycles * (gamma + 1)), dtype=torch.int32, device=dev),
                   n_emitted=torch.empty(R, dtype=torch.int32, device=dev),
                   stats=torch.empty(2 * gamma + 3, dtype=torch.int64, device=dev))
    nbytes = decode_workspace_bytes(R, gamma, V, r, d, dt)
    if nbytes == 0:
        raise DsparkError("dspark_decode_workspace_bytes", EINVAL)
    ws = _ws(nbytes, dev, ws)
    rc = lib().dspark_decode_run(R, gamma, V, r, d, dt, ncycles, _p(Ub), _p(Hb), _p(W1),
                                 _p(W2t), _p(w), _p(temps), _p(Tb), _p(x0), policy,
                                 float(threshold), _p(sps), sps_B0,
                                 0 if sps is None else sps.numel(), seed, _p(out["tokens"]),
                                 _p(out["n_emitted"]), _p(out["stats"]), _p(status), _p(ws),
                                 ws.numel() * ws.element_size(), _stream())
    _raise("dspark_decode_run", rc)
    return out


def sps_profile(target, U, W2t, bias_rows, x, lse, logit_x, B_list, reps=10, *, ws=None,
                status=None, ell=None):
    """SPS(B) at the profiled batches B_list: the verification pass timed as the stand-in
    engine (steps/s).  Operands as verify(); returns a numpy float32 array [len(B_list)].
    ell: optional [R] int32 device tensor that receives the lengths of the last profiled
    batch.  Synchronises with the current stream."""
    import numpy as np
    torch = _torch()
    _chk(U, "U")
    R, gamma, V = U.shape
    dt = _dt(U)
    r = W2t.shape[1]
    _chk(target, "target", (R, gamma + 1, V), U.dtype)
    _chk(bias_rows, "bias_rows", (R, gamma, r))
    bl = np.ascontiguousarray(np.asarray(B_list, dtype=np.int32))
    sps = np.zeros(bl.size, np.float32)
    dev = U.device
    if ell is None:
        ell = torch.empty(R, dtype=torch.int32, device=dev)
    _chk(ell, "ell", (R,), torch.int32)
    n_acc = torch.empty(R, dtype=torch.int32, device=dev)
    y = torch.empty((R, gamma + 1), dtype=torch.int32, device=dev)
    cs = torch.empty((R, gamma), dtype=torch.float32, device=dev)
    ws = _ws(verify_workspace_bytes(R, gamma, V, r), dev, ws)
    rc = lib().dspark_sps_profile(R, gamma, V, r, dt, _p(target), _p(U), _p(W2t),
                                  _p(bias_rows), _dt(bias_rows), _p(x), _p(lse), _p(logit_x),
                                  bl.size, bl.ctypes.data_as(C.c_void_p), reps,
                                  sps.ctypes.data_as(C.c_void_p), _p(ell), _p(n_acc), _p(y),
                                  _p(cs), _p(status), _p(ws), ws.numel() * ws.element_size(),
                                  _stream())
    _raise("dspark_sps_profile", rc)
    return sps


def sps_interpolate(B_list, sps_at, B0, B1):
    """The SPS table for B = B0 .. B1 from profiled points (host only)."""
    import numpy as np
    bl = np.ascontiguousarray(np.asarray(B_list, dtype=np.int32))
    sa = np.ascontiguousarray(np.asarray(sps_at, dtype=np.float32))
    if bl.shape != sa.shape:
        raise ValueError("B_list and sps_at differ in length")
    out = np.zeros(max(B1 - B0 + 1, 0), np.float32)
    rc = lib().dspark_sps_interpolate(bl.size, bl.ctypes.data_as(C.c_void_p),
                                      sa.ctypes.data_as(C.c_void_p), B0, B1,
                                      out.ctypes.data_as(C.c_void_p))
    _raise("dspark_sps_interpolate", rc)
    return out
