"""Pins of the oracle's gate, provenance and packing (CPU only).

The gate is pinned by hand-built rows with exact rational ratios, by scale invariance,
by a math.fsum brute force and by the special thresholds; provenance by an exhaustive
comparison with an independent nearest-recomputing-ancestor search over every small
first-parent graph and every mask; packing by its count/ordering invariants."""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import bruteforce_provenance, fold_state, gate, pack, resolve
from synth import BUDGETS, CONFIGS, budget_config, custom_config, graph_depth, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _two_node(parent, child):
    H = np.array([[parent], [child]], dtype=np.float32)       # [N=2, B=1, d]
    return H, np.array([-1, 0], dtype=np.int32)


def test_gate_hand_built_rows():
    spec = json.load(open(os.path.join(GOLDEN, "gate_cases.json")))
    tau = spec["tau"]
    for case in spec["cases"]:
        H, fs = _two_node(case["parent"], case["child"])
        r32, r64, rec = gate(H, fs, tau)
        want = math.inf if case["r_den"] == 0 else case["r_num"] / case["r_den"]
        if math.isinf(want):
            assert math.isinf(r64[1, 0]) and math.isinf(r32[1, 0])
        else:
            assert r64[1, 0] == pytest.approx(want, rel=1e-15, abs=0)
            assert r32[1, 0] == pytest.approx(want, rel=1e-6, abs=0)
        assert bool(rec[1, 0]) == case["recompute"], case
        assert rec[0, 0] and math.isinf(r32[0, 0])             # the root never folds


def test_gate_matches_fsum_bruteforce_and_scale_invariance():
    rng = np.random.default_rng(3)
    H = rng.standard_normal((5, 6, 48)).astype(np.float32)
    H[3, 2] = H[1, 2]                                          # an identical row
    fs = np.array([-1, 0, 1, 1, 0], dtype=np.int32)
    r32, r64, _ = gate(H, fs, 0.1)
    for n in range(1, 5):
        for i in range(6):
            c = [float(v) for v in H[n, i]]
            p = [float(v) for v in H[fs[n], i]]
            num = math.sqrt(math.fsum((a - b) ** 2 for a, b in zip(c, p)))
            den = math.sqrt(math.fsum(b * b for b in p))
            assert r64[n, i] == pytest.approx(num / den, rel=1e-13)
            assert r32[n, i] == pytest.approx(num / den, rel=2e-6)
    assert r32[3, 2] == 0 and r64[3, 2] == 0
    # powers of two scale both norms exactly
    r32b, r64b, _ = gate(H * np.float32(8.0), fs, 0.1)
    np.testing.assert_array_equal(r64b, r64)
    np.testing.assert_array_equal(r32b, r32)


def test_gate_special_thresholds():
    w = make_workload(CONFIGS[0])
    _, _, rec_neg = gate(w.H, w.fold_src, -1.0)
    assert rec_neg.all()                                        # tau < 0: dense
    _, _, rec_inf = gate(w.H, w.fold_src, math.inf)
    assert rec_inf[0].all() and not rec_inf[1:].any()           # tau = inf: fold all children
    H = w.H.copy()
    H[2, 5, 0] = np.nan
    _, _, rec_nan = gate(H, w.fold_src, math.inf)
    assert rec_nan[2, 5]                                        # NaN ratio recomputes
    _, _, rec_nan_tau = gate(w.H, w.fold_src, math.nan)
    assert rec_nan_tau.all()                                    # NaN tau: nothing folds


def test_gate_ratio_peaks_at_revealed_positions():
    """Workload sanity: the largest difference sits at the revealed positions and the
    ripple decays with distance from them (the 'residual ripple' the pages describe)."""
    w = make_workload(CONFIGS[1], weights=False)
    r32, r64, _ = gate(w.H, w.fold_src, 0.05)
    B = w.cfg.block
    by_dist = {}
    for n in range(1, w.cfg.num_nodes):
        rev = w.reveals[n]
        assert set(np.argsort(-r64[n])[: len(rev)]) == set(rev)
        dist = np.min(np.abs(np.arange(B)[:, None] - rev[None, :]), axis=1)
        for i in range(B):
            by_dist.setdefault(int(dist[i]), []).append(r64[n, i])
    means = [np.mean(by_dist[k]) for k in sorted(by_dist) if k <= 8]
    assert all(a > b for a, b in zip(means, means[1:]))


def test_recompute_count_monotone_in_tau():
    w = make_workload(CONFIGS[2], weights=False)
    Ks = [fold_state(w.H, w.fold_src, t)["K"] for t in (-1, 0.0, 0.02, 0.05, 0.1, 1.0, math.inf)]
    assert all(a >= b for a, b in zip(Ks, Ks[1:]))
    assert Ks[0] == w.cfg.slots and Ks[-1] == w.cfg.block


def _all_first_parent_graphs(N):
    for choice in itertools.product(*[range(n) for n in range(1, N)]):
        yield np.array([-1] + list(choice), dtype=np.int32)


@pytest.mark.parametrize("N,B", [(2, 3), (3, 3), (4, 3), (5, 2)])
def test_provenance_exhaustive_small_graphs(N, B):
    for fs in _all_first_parent_graphs(N):
        for bits in range(1 << ((N - 1) * B)):
            rec = np.ones((N, B), dtype=bool)
            for n in range(1, N):
                for i in range(B):
                    rec[n, i] = bool((bits >> ((n - 1) * B + i)) & 1)
            src = resolve(rec, fs)
            np.testing.assert_array_equal(src, bruteforce_provenance(rec, fs))


def test_provenance_random_deep_dags():
    rng = np.random.default_rng(11)
    for trial in range(40):
        cfg = custom_config(num_nodes=int(rng.integers(2, 40)), block=int(rng.integers(1, 9)),
                            graph=["dag", "dag_deep", "chain", "tree3"][trial % 4],
                            seed=trial, max_depth=6)
        from synth.workload import draft_graph
        fs, _ = draft_graph(cfg, np.random.default_rng(trial))
        rec = rng.random((cfg.num_nodes, cfg.block)) < rng.random()
        rec[0] = True
        np.testing.assert_array_equal(resolve(rec, fs), bruteforce_provenance(rec, fs))


def test_provenance_special_cases():
    w = make_workload(CONFIGS[4], weights=False)
    N, B = w.cfg.num_nodes, w.cfg.block
    assert graph_depth(w.fold_src).max() == 6
    st = fold_state(w.H, w.fold_src, -1.0)
    np.testing.assert_array_equal(st["src"], np.repeat(np.arange(N)[:, None], B, axis=1))
    st = fold_state(w.H, w.fold_src, math.inf)
    np.testing.assert_array_equal(st["src"], np.zeros((N, B), dtype=np.int32))


@pytest.mark.parametrize("cfg_id", [0, 1, 2])
def test_pack_invariants(cfg_id):
    w = make_workload(CONFIGS[cfg_id], weights=False)
    N, B = w.cfg.num_nodes, w.cfg.block
    st = fold_state(w.H, w.fold_src, w.cfg.tau)
    rec, src = st["recompute"], st["src"]
    ps, sr, K = st["packed_slot"], st["slot_row"], st["K"]
    # packed count = root rows + child rows over tau
    assert K == B + int(np.sum(~(st["r32"][1:] <= np.float32(w.cfg.tau))))
    assert K == int(rec.sum())
    assert np.all(np.diff(ps) > 0)                              # ascending, unique
    assert np.all(rec.reshape(-1)[ps])
    for n in range(N):
        for i in range(B):
            k = sr[n, i]
            assert 0 <= k < K
            assert ps[k] == src[n, i] * B + i                       # same position,
            assert rec[src[n, i], i]                               # a recompute slot
    # and the brute-force rank definition
    order = {s: k for k, s in enumerate(sorted(int(s) for s in np.flatnonzero(rec)))}
    for n in range(N):
        for i in range(B):
            assert sr[n, i] == order[int(src[n, i]) * B + i]


def test_budget_sweep_fold_states_nest():
    """The draft-budget sweep grows one 3-ary level-order tree: each smaller budget's graph,
    hidden states and fold decisions are the first nodes of the next one's, so the packed
    count never falls as branches are added, and every budget keeps the pack invariant."""
    prev = None
    for n in BUDGETS:
        cfg = budget_config(n)
        w = make_workload(cfg, weights=False)
        assert list(w.fold_src[1:]) == [(m - 1) // 3 for m in range(1, n)]
        st = fold_state(w.H, w.fold_src, cfg.tau)
        B = cfg.block
        assert st["K"] == B + int(np.sum(~(st["r32"][1:] <= np.float32(cfg.tau))))
        assert fold_state(w.H, w.fold_src, -1.0)["K"] == cfg.slots
        if prev is not None:
            pn, pH, prec, pK = prev
            np.testing.assert_array_equal(w.H[:pn], pH)
            np.testing.assert_array_equal(st["recompute"][:pn], prec)
            assert st["K"] >= pK
        prev = (n, w.H, st["recompute"], st["K"])
    assert budget_config(16) == CONFIGS[1].with_(name=budget_config(16).name)


def test_pack_edge_cases():
    rec = np.ones((1, 5), dtype=bool)                          # root only
    src = resolve(rec, np.array([-1], dtype=np.int32))
    ps, sr, K = pack(rec, src)
    assert K == 5 and list(ps) == [0, 1, 2, 3, 4] and list(sr[0]) == [0, 1, 2, 3, 4]
    rec = np.zeros((3, 4), dtype=bool)
    rec[0] = True
    fs = np.array([-1, 0, 1], dtype=np.int32)
    ps, sr, K = pack(rec, resolve(rec, fs))
    assert K == 4 and (sr == np.arange(4)[None, :]).all()


def test_golden_tiny_layer_regression():
    """The oracle still reproduces the fixture its own script wrote (drift guard)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(GOLDEN, "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    want = json.load(open(os.path.join(GOLDEN, "tiny_layer.json")))
    got = mod.compute()
    for key in ("fold_src", "recompute", "src", "slot_row", "K"):
        assert got[key] == want[key], key
    np.testing.assert_allclose(got["y_row_sums"], want["y_row_sums"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got["y_first8"], want["y_first8"], rtol=1e-12, atol=1e-12)
