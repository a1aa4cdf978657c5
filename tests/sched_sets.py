"""Confidence sets and SPS tables for the scheduler's parity and reading tests: workload-
shaped Beta confidences, and adversarial sets (exact 1.0s and 0s, subnormal running
products, massive cross-request ties, a single request, a ragged shape)."""
import numpy as np

from draft_sampling_scheduling_amd import synth


def _conf_sets():
    rng = np.random.default_rng(42)
    out = []
    out.append(("beta-c3", rng.beta(6, 1.6, (256, 8)).astype(np.float32), 1, "c3"))
    c = rng.choice(np.array([1.0, 1.0, 1.0, 0.5, 0.0, 0.999], np.float32), (100, 8))
    out.append(("exact-ones-zeros", c, 1, "smooth"))
    c = np.full((64, 16), 0.02, np.float32)
    c[::3] = 1e-10  # subnormal running products
    out.append(("subnormal", c, 1, "smooth"))
    out.append(("all-equal", np.full((300, 5), 0.9, np.float32), 1, "smooth"))
    c = rng.beta(8, 1.5, (512, 16)).astype(np.float32)
    c[1::2] = rng.beta(2, 2, (256, 16))
    out.append(("c4-size", c, 1, "c4"))
    out.append(("R1", np.array([[0.8, 0.9]], np.float32), 1, "appendix"))
    out.append(("ragged-37x7", rng.uniform(0, 1, (37, 7)).astype(np.float32), 1, "smooth"))
    return out


def _sps(kind, R, gamma):
    B = np.arange(1, R * (gamma + 1) + 1, dtype=np.float64)
    if kind == "appendix":
        return np.array([1.0, 0.5, 0.45], np.float32), 1
    if kind == "c4":
        cfg = synth.CONFIGS["c4"]
        return synth.sps_table(cfg), cfg.sps_B0
    if kind == "c3":
        cfg = synth.CONFIGS["c3"]
        return synth.sps_table(cfg), cfg.sps_B0
    return (1.0 / (1.0 + 0.01 * B + 0.03 * np.floor(B / 37))).astype(np.float32), 1
