"""Helpers shared by the parity tests: oracle runs, tie-band handling, error metrics."""
import math

import numpy as np

from oracle import fold_state, layer

# Tolerances on the layer output: max|y - y_ref| / max|y_ref|.
TOL = {"f32": 1e-3, "bf16": 2e-2}
# Slots whose ratio lies within this relative distance of tau may decide either way.
BAND = 1e-4


def max_abs_rel(got: np.ndarray, ref: np.ndarray) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def band(r64: np.ndarray, tau: float) -> np.ndarray:
    """Slots excluded from the bit-exact mask comparison."""
    if not (0 < tau < math.inf):
        return np.zeros(r64.shape, dtype=bool)
    return np.abs(r64 - tau) <= BAND * tau


def oracle_state(w, tau):
    return fold_state(w.H, w.fold_src, tau)


def oracle_layer(w, tau, state=None, slots=None, layer_idx=0, H=None, attn="correct"):
    cfg = w.cfg
    pk, pv = w.prefix_kv(layer_idx)
    return layer(w.weights[layer_idx], w.H if H is None else H, w.fold_src, tau, pk, pv,
                 n_q=cfg.n_q, n_kv=cfg.n_kv, eps=cfg.rms_eps, state=state, slots=slots,
                 attn=attn, rope_theta=cfg.rope_theta)


def assert_fold_state_equal(gpu, ora, tau, ratio_rtol=2e-5):
    """Masks bit-exact outside the tie band; ratios close; provenance and packing
    bit-exact when the masks agree everywhere.  Returns True if the masks agree."""
    excl = band(ora["r64"], tau)
    rec_g, rec_o = gpu["recompute"], ora["recompute"]
    mism = (rec_g != rec_o) & ~excl
    assert not mism.any(), f"mask mismatch outside the tie band at {np.argwhere(mism)[:8]}"
    finite = np.isfinite(ora["r64"])
    np.testing.assert_array_equal(np.isfinite(gpu["ratio"]), finite)
    np.testing.assert_allclose(gpu["ratio"][finite], ora["r64"][finite], rtol=ratio_rtol,
                               atol=1e-7)
    if (rec_g == rec_o).all():
        np.testing.assert_array_equal(gpu["src"], ora["src"])
        assert gpu["K"] == ora["K"]
        np.testing.assert_array_equal(gpu["packed_slot"], ora["packed_slot"])
        np.testing.assert_array_equal(gpu["slot_row"], ora["slot_row"])
        return True
    return False
