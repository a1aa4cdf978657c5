"""Seeded synthetic inputs for the draft -> schedule -> verify path.

This module is the only code the HIP path and the CPU oracle's tests share: it draws random
inputs and holds none of the method's arithmetic.  Everything is numpy (PCG64), seeded per
config, per operand and per request, so any subset of requests can be regenerated on its
own, bit for bit.

The shapes and value laws are the five workloads the path is exercised on (the pages
measure on public benchmarks with trained models; these synthetic tensors stand in for the
backbone's outputs U_k, h_k, the head's weights and the target model):

  c1  tiny Markov cycle, fp32     R=4   gamma=4  V=1024   r=16  d=64
  c2  Markov mid-size, bf16       R=64  gamma=8  V=32000  r=256 d=2560
  c3  Markov headline, bf16       R=256 gamma=8  V=151936 r=256 d=4096
  c4  scheduler stress, bf16      R=512 gamma=16 V=151936 r=256 d=5120
  c5  RNN head + async scheduler  R=256 gamma=16 V=129280 r=256 d=4096

bf16 operands are produced as uint16 bit patterns rounded once, to nearest-even, from the
float32 draw; both sides read exactly those bits.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


# --------------------------------------------------------------------------------------
# bf16 helpers (encoding only)
# --------------------------------------------------------------------------------------
def bf16_bits(x) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    b = f.view(np.uint32)
    r = (b >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += b  # finite inputs: no 32-bit overflow
    r >>= 16
    return r.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Widen uint16 bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


# --------------------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    seed: int
    R: int
    gamma: int
    V: int
    r: int
    d: int
    dtype: str             # "f32" or "bf16"
    head: str              # "markov" or "rnn"
    u_law: str             # "normal", "zipf", "mixed"
    u_scale: float         # std of U for "normal"
    weight_std: float | None  # W1, W2 (and W_gco) std; None = 1/sqrt(r) (W_gco: 1/sqrt(2r+d))
    h_std: float
    w_std: float | None    # confidence weights std; None = sqrt(1/(d+r))
    target_noise: float    # std of the target's deviation from the draft logits
    sps_kind: str          # "c1", "smooth", "staircase"
    sps_alpha: float
    sps_B0: int
    sps_B1: int            # inclusive
    sched_mode: int        # 0 sync+break, 1 global, 2 async lag-2

    @property
    def is_bf16(self) -> bool:
        return self.dtype == "bf16"


CONFIGS = {
    "c1": Config("c1", 1, 4, 4, 1024, 16, 64, "f32", "markov", "normal", 1.5, 0.1, 1.0, 0.05,
                 0.5, "smooth", 0.02, 1, 20, 0),
    "c2": Config("c2", 2, 64, 8, 32000, 256, 2560, "bf16", "markov", "normal", 2.0, None, 1.0,
                 None, 0.7, "smooth", 0.004, 64, 576, 0),
    "c3": Config("c3", 3, 256, 8, 151936, 256, 4096, "bf16", "markov", "zipf", 1.0, None, 1.0,
                 None, 0.6, "smooth", 0.002, 256, 2304, 0),
    "c4": Config("c4", 4, 512, 16, 151936, 256, 5120, "bf16", "markov", "mixed", 1.0, None,
                 1.0, None, 0.0, "staircase", 0.0005, 512, 8704, 1),
    "c5": Config("c5", 5, 256, 16, 129280, 256, 4096, "bf16", "rnn", "zipf", 1.0, None, 1.0,
                 None, 0.6, "staircase", 0.0005, 256, 4352, 2),
}


def scaled(cfg: Config, **kw) -> Config:
    """The same value laws at other sizes (tests use small and ragged shapes)."""
    return dataclasses.replace(cfg, **kw)


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


def _encode(cfg: Config, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return bf16_bits(x) if cfg.is_bf16 else x


def _wstd(cfg: Config) -> float:
    return cfg.weight_std if cfg.weight_std is not None else 1.0 / math.sqrt(cfg.r)


def _u_row_law(cfg: Config, req: int):
    """(kind, scale) of request req's U rows; "mixed" interleaves two regimes."""
    if cfg.u_law == "mixed":
        return ("normal", 4.0) if req % 2 == 0 else ("normal", 1.0)
    return (cfg.u_law, cfg.u_scale)


def _u_rows(cfg: Config, rng: np.random.Generator, req: int, n: int) -> np.ndarray:
    kind, scale = _u_row_law(cfg, req)
    if kind == "zipf":
        # Zipf(1.1)-ranked logits: -1.1 ln(rank), ranks a fresh random permutation per row
        base = (-1.1 * np.log(np.arange(1, cfg.V + 1, dtype=np.float64))).astype(np.float32)
        out = np.empty((n, cfg.V), np.float32)
        for i in range(n):
            out[i] = base[rng.permutation(cfg.V)]
        out += rng.standard_normal((n, cfg.V), dtype=np.float32)
        return out
    return rng.standard_normal((n, cfg.V), dtype=np.float32) * np.float32(scale)


def anchors(cfg: Config) -> np.ndarray:
    return _rng(cfg.seed, 0).integers(0, cfg.V, cfg.R).astype(np.int32)


def _map(fn, items):
    """fn over items on a thread pool (numpy releases the GIL); order kept."""
    items = list(items)
    if len(items) < 4:
        return [fn(i) for i in items]
    import concurrent.futures as cf
    import os
    workers = min(16, os.cpu_count() or 1, len(items))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def U_rows(cfg: Config, reqs) -> np.ndarray:
    """U[reqs] as [len(reqs)][gamma][V] (encoded)."""
    out = _map(lambda q: _encode(cfg, _u_rows(cfg, _rng(cfg.seed, 1, q), q, cfg.gamma)), reqs)
    if not out:
        return _encode(cfg, np.zeros((0, cfg.gamma, cfg.V), np.float32))
    return np.stack(out)


def h_rows(cfg: Config, reqs) -> np.ndarray:
    out = [_rng(cfg.seed, 2, q).standard_normal((cfg.gamma, cfg.d), dtype=np.float32)
           * np.float32(cfg.h_std) for q in reqs]
    return _encode(cfg, np.stack(out) if out else np.zeros((0, cfg.gamma, cfg.d), np.float32))


def weights(cfg: Config) -> dict:
    """W1 [V][r], W2 [r][V] (the pages' layout), w [d+r] fp32, W_gco [3r][2r+d] (rnn)."""
    s = np.float32(_wstd(cfg))

    def draw(key_shape):
        key, shape = key_shape
        return _encode(cfg, _rng(cfg.seed, key).standard_normal(shape, dtype=np.float32) * s)

    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(max_workers=2) as ex:
        W1, W2 = ex.map(draw, [(3, (cfg.V, cfg.r)), (4, (cfg.r, cfg.V))])
    wstd = cfg.w_std if cfg.w_std is not None else math.sqrt(1.0 / (cfg.d + cfg.r))
    w = _rng(cfg.seed, 5).standard_normal(cfg.d + cfg.r, dtype=np.float32) * np.float32(wstd)
    out = dict(W1=W1, W2=W2, w=w)
    if cfg.head == "rnn":
        K = 2 * cfg.r + cfg.d
        gs = np.float32(cfg.weight_std if cfg.weight_std is not None else 1.0 / math.sqrt(K))
        out["W_gco"] = _encode(cfg, _rng(cfg.seed, 6).standard_normal((3 * cfg.r, K),
                                                                      dtype=np.float32) * gs)
    return out


def sps_table(cfg: Config) -> np.ndarray:
    """SPS(B) for B = sps_B0 .. sps_B1 (float32): engine steps/s against verify batch."""
    B = np.arange(cfg.sps_B0, cfg.sps_B1 + 1, dtype=np.float64)
    if cfg.sps_kind == "staircase":
        v = 1.0 / (1.0 + cfg.sps_alpha * B + 0.02 * np.floor((B + 64) / 128))
    else:
        v = 1.0 / (1.0 + cfg.sps_alpha * B)
    return v.astype(np.float32)


def inputs(cfg: Config) -> dict:
    """All draft inputs of a config (numpy, encoded)."""
    reqs = range(cfg.R)
    out = dict(U=U_rows(cfg, reqs), h=h_rows(cfg, reqs), x0=anchors(cfg), sps=sps_table(cfg))
    out.update(weights(cfg))
    return out


def target_noise_std(cfg: Config, req: int) -> float:
    if cfg.u_law == "mixed":
        return 0.3 if req % 2 == 0 else 1.0
    return cfg.target_noise


def target_parts(cfg: Config, reqs, cycle: int):
    """Pieces of the synthetic target-model stand-in for one cycle.

    Returns (noise [n][gamma+1][V] float32, fresh [n][V] float32): target row j (1..gamma)
    is the draft's logits at position j plus noise[:, j-1]; the bonus row gamma+1 is
    fresh + noise[:, gamma] (a new U-law row, no head bias).  The caller adds and encodes.
    """
    noise, fresh = [], []
    for q in reqs:
        g = _rng(cfg.seed, 10, cycle, q)
        noise.append(g.standard_normal((cfg.gamma + 1, cfg.V), dtype=np.float32)
                     * np.float32(target_noise_std(cfg, q)))
        fresh.append(_u_rows(cfg, _rng(cfg.seed, 11, cycle, q), q, 1)[0])
    n = len(noise)
    return (np.stack(noise) if n else np.zeros((0, cfg.gamma + 1, cfg.V), np.float32),
            np.stack(fresh) if n else np.zeros((0, cfg.V), np.float32))


def encode(cfg: Config, x) -> np.ndarray:
    """Encode float values in the config's operand type (bf16 bits or float32)."""
    return _encode(cfg, x)


def decode(cfg: Config, a) -> np.ndarray:
    """Operand values as float32 (bf16 widened exactly)."""
    return bf16_to_f32(a) if cfg.is_bf16 else np.ascontiguousarray(a, dtype=np.float32)


def sts_heldout(N: int, temps, seed: int, loc: float = 1.5, scale: float = 2.0):
    """Held-out calibration samples for the STS fit: confidence logits z [N][gamma] float32,
    z ~ N(loc, scale^2), and accepted lengths n_acc [N] int32 drawn from a chain in which
    position k is accepted, given its prefix was, with probability sigmoid(z_k / temps[k]).
    The running product of those probabilities is then the calibrated prefix predictor,
    so a correct fit recovers `temps` (up to the grid step and sampling noise)."""
    rng = np.random.default_rng([0x575, seed])
    gamma = len(temps)
    z = rng.normal(loc, scale, (N, gamma)).astype(np.float32)
    p = 1.0 / (1.0 + np.exp(-z.astype(np.float64) / np.asarray(temps, np.float64)))
    ok = rng.uniform(size=(N, gamma)) < p
    n_acc = np.where(ok.all(axis=1), gamma, np.argmin(ok, axis=1)).astype(np.int32)
    return z, n_acc


def train_batch(cfg: Config) -> dict:
    """Teacher-forced training blocks for the loss forward: target logits [R][gamma][V]
    (a fresh U-law row of the request plus the config's target noise, encoded) and the
    reference tokens x*_1..x*_gamma [R][gamma] int32, the argmax of each target row (a
    greedy target continuation).  x*_0 is the request's anchor."""
    T = np.empty((cfg.R, cfg.gamma, cfg.V), np.float32)
    for q in range(cfg.R):
        g = _rng(cfg.seed, 12, q)
        T[q] = _u_rows(cfg, g, q, cfg.gamma)
        T[q] += g.standard_normal((cfg.gamma, cfg.V), dtype=np.float32) * np.float32(
            max(target_noise_std(cfg, q), 0.1))
    xstar = np.argmax(T, axis=2).astype(np.int32)
    return dict(target=_encode(cfg, T), xstar=xstar)


def toy_chain(V: int, gamma: int, r: int, d: int, R: int, seed: int, dtype: str = "bf16",
              sps_alpha: float = 0.002) -> dict:
    """A toy decode chain for the multi-cycle driver.  Target: a bigram model whose logits
    after token t are Tb[t] = a Zipf(1.1)-ranked row (one ranking shared by all t) + N(0, 1).
    Backbone stand-in: U_k for anchor a is Ub[a][k-1] = Tb[a] + N(0, (0.3 + 0.2 k)^2), a base
    prediction that drifts from the anchor's next-token law further into the block; h rows
    N(0, 1).  Head weights as the configs (std 1/sqrt(r); w std sqrt(1/(d+r))).  Anchors
    uniform; SPS(B) = 1/(1 + sps_alpha B) for B = 1 .. R(gamma+1)."""
    cfg = Config("toy", seed, R, gamma, V, r, d, dtype, "markov", "zipf", 1.0, None, 1.0,
                 None, 1.0, "smooth", sps_alpha, 1, R * (gamma + 1), 0)
    g = _rng(0x70, seed)
    base = (-1.1 * np.log(np.arange(1, V + 1, dtype=np.float64))).astype(np.float32)
    Tb = base[g.permutation(V)][None, :] + g.standard_normal((V, V), dtype=np.float32)
    sig = (0.3 + 0.2 * np.arange(1, gamma + 1, dtype=np.float32))[None, :, None]
    Ub = Tb[:, None, :] + g.standard_normal((V, gamma, V), dtype=np.float32) * sig
    Hb = g.standard_normal((V, gamma, d), dtype=np.float32)
    s = np.float32(1.0 / math.sqrt(r))
    W1 = g.standard_normal((V, r), dtype=np.float32) * s
    W2 = g.standard_normal((r, V), dtype=np.float32) * s
    w = g.standard_normal(d + r, dtype=np.float32) * np.float32(math.sqrt(1.0 / (d + r)))
    x0 = g.integers(0, V, R).astype(np.int32)
    B = np.arange(1, R * (gamma + 1) + 1, dtype=np.float64)
    return dict(Tb=_encode(cfg, Tb), Ub=_encode(cfg, Ub), Hb=_encode(cfg, Hb),
                W1=_encode(cfg, W1), W2=_encode(cfg, W2), w=w, x0=x0,
                sps=(1.0 / (1.0 + sps_alpha * B)).astype(np.float32), sps_B0=1)
