"""Pins of the oracle's LM head + per-branch argmax (the step after the layer stack).

Each check is independent of the oracle's own matrix product: an fsum brute force, an
identity head whose argmax is the argmax of the normalised row itself, a permuted
vocabulary, the first-index tie rule, and the folding semantics at tau = +inf / tau < 0."""
import math

import numpy as np
import pytest

from oracle import fold_state, lm_head_argmax
from synth import custom_config, lm_head_weights, make_workload


def _tiny(seed=3, N=4, B=5, d=8, V=11):
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((N, B, d))
    fs = np.array([-1] + [(m - 1) // 3 for m in range(1, N)], dtype=np.int32)
    w = rng.standard_normal((V, d))
    g = rng.uniform(0.5, 1.5, d)
    return y, fs, w, g


def test_bruteforce_fsum_loops():
    y, fs, w, g = _tiny()
    st = fold_state(y, fs, 0.9)
    out = lm_head_argmax(y, g, w, st, eps=1e-6)
    N, B, d = y.shape
    flat = y.reshape(N * B, d)
    for k, slot in enumerate(st["packed_slot"]):
        x = [float(v) for v in flat[slot]]
        r = math.sqrt(math.fsum(v * v for v in x) / d + 1e-6)
        a = [x[j] / r * float(g[j]) for j in range(d)]
        logits = [math.fsum(a[j] * float(w[v, j]) for j in range(d)) for v in range(len(w))]
        best = 0
        for v in range(1, len(logits)):
            if logits[v] > logits[best]:
                best = v
        assert out["row_token"][k] == best
        assert abs(out["row_logit"][k] - logits[best]) <= 1e-12 * max(1.0, abs(logits[best]))
    for n in range(N):
        for i in range(B):
            assert out["token"][n, i] == out["row_token"][st["slot_row"][n, i]]


def test_identity_head_takes_argmax_of_the_row():
    # w_lm = 3 I (vocab = d) and g = 1: the logits are the normalised row times 3, whose
    # argmax is the row's own argmax (RMS scaling is a positive factor)
    y, fs, _, _ = _tiny(seed=5, d=16, V=16)
    st = fold_state(y, fs, -1.0)                  # dense: every slot packed
    out = lm_head_argmax(y, np.ones(16), 3.0 * np.eye(16), st, eps=1e-6)
    np.testing.assert_array_equal(out["token"], np.argmax(y, axis=2))


def test_permuted_vocabulary_permutes_tokens():
    y, fs, w, g = _tiny(seed=7, V=23)
    st = fold_state(y, fs, 0.5)
    perm = np.random.default_rng(1).permutation(len(w))
    base = lm_head_argmax(y, g, w, st, eps=1e-6)
    moved = lm_head_argmax(y, g, w[perm], st, eps=1e-6)
    inv = np.argsort(perm)
    np.testing.assert_array_equal(moved["row_token"], inv[base["row_token"]])
    np.testing.assert_allclose(moved["row_logit"], base["row_logit"], rtol=0, atol=1e-12)


def test_ties_take_the_lowest_index():
    # exact arithmetic, so ties are true ties whatever the summation order: rows of +-2 with
    # eps = 0 normalise to exactly +-1, integer weights give integer logits
    rng = np.random.default_rng(9)
    N, B, d, V = 3, 4, 8, 6
    y = 2.0 * rng.choice([-1.0, 1.0], size=(N, B, d))
    fs = np.array([-1, 0, 0], dtype=np.int32)
    w = rng.integers(-3, 4, size=(V, d)).astype(np.float64)
    st = fold_state(y, fs, -1.0)
    base = lm_head_argmax(y, np.ones(d), w, st, eps=0.0)
    # the loop below is the definition: first index of the maximum
    flat = np.sign(y.reshape(N * B, d))
    for k, slot in enumerate(st["packed_slot"]):
        lg = [int(sum(int(flat[slot, j]) * int(w[v, j]) for j in range(d))) for v in range(V)]
        assert base["row_token"][k] == lg.index(max(lg))
    # every vocabulary row duplicated after the originals: v and v + V tie, v wins
    dup = lm_head_argmax(y, np.ones(d), np.concatenate([w, w]), st, eps=0.0)
    np.testing.assert_array_equal(dup["row_token"], base["row_token"])
    # the winner's row copied to the front: the copy (index 0) wins
    for k, t in enumerate(base["row_token"]):
        w2 = np.concatenate([w[t:t + 1], w])
        assert lm_head_argmax(y, np.ones(d), w2, st, eps=0.0, rows=[k])["row_token"][k] == 0


def test_folding_semantics():
    y, fs, w, g = _tiny(seed=11, N=7, B=4)
    dense = lm_head_argmax(y, g, w, fold_state(y, fs, -1.0), eps=1e-6)
    inf = lm_head_argmax(y, g, w, fold_state(y, fs, math.inf), eps=1e-6)
    # tau = inf: only the root computes; every branch predicts the root's tokens
    for n in range(y.shape[0]):
        np.testing.assert_array_equal(inf["token"][n], dense["token"][0])
    # tau < 0: each slot's own row
    for n in range(y.shape[0]):
        one = lm_head_argmax(y[n:n + 1], g, w, fold_state(y[n:n + 1], fs[:1], -1.0), eps=1e-6)
        np.testing.assert_array_equal(dense["token"][n], one["token"][0])


def test_row_subset_equals_full():
    cfg = custom_config(name="lm-subset", num_nodes=6, block=8, hidden=64, dtype="bf16",
                        seed=21)
    w = make_workload(cfg, weights=False)
    g, wl = lm_head_weights(cfg, 300)
    st = fold_state(w.H, w.fold_src, 0.05)
    full = lm_head_argmax(w.H, g, wl, st, eps=1e-6)
    part = lm_head_argmax(w.H, g, wl, st, eps=1e-6, rows=[0, st["K"] - 1])
    for k in (0, st["K"] - 1):
        assert part["row_token"][k] == full["row_token"][k]
        assert abs(part["row_logit"][k] - full["row_logit"][k]) <= 1e-12 * abs(full["row_logit"][k])


def test_lm_head_weights_seeded_and_rounded():
    cfg = custom_config(name="lm-w", hidden=64, dtype="bf16", seed=4)
    g1, w1 = lm_head_weights(cfg, 100)
    g2, w2 = lm_head_weights(cfg, 100)
    np.testing.assert_array_equal(w1, w2)
    assert np.all(g1 == 1.0)
    assert np.all((w1.view(np.uint32) & 0xFFFF) == 0)          # bf16-representable
    assert abs(float(np.std(w1)) - cfg.weight_std) < 0.002
