"""Pins of the oracle's layer stack and its bf16 hand-over between layers (CPU only).

  * round_to_bf16 equals torch's float32 -> bfloat16 conversion (round to nearest even)
    on fp32 inputs, and a brute-force nearest-neighbour search on float64 inputs;
  * with nothing folded, the stack equals textbook dense layers (torch CPU library
    routines) chained with each layer's own weights and prefix;
  * at finite tau it equals the chain of textbook layers on substituted inputs where
    every layer re-runs the pinned gate/provenance/packing on its own input -- the
    workloads are chosen so that the recompute set really changes between layers;
  * tau = +inf keeps every child's offset from the root exactly, through all layers."""
import math

import numpy as np
import pytest
import torch

from oracle import fold_state, round_to_bf16, stack
from synth import custom_config, make_workload

from test_oracle_layer import torch_dense

# weights stronger than the benchmark's 0.02 so that every layer moves the child/parent
# ratios enough to change the recompute set
STACKS = [
    custom_config(num_nodes=6, block=8, hidden=64, n_q=2, n_kv=1, head_dim=64, ffn=128,
                  prefix=16, graph="tree3", reveal=(1, 2), layers=4, seed=31, weight_std=0.15),
    custom_config(num_nodes=7, block=5, hidden=128, n_q=4, n_kv=2, head_dim=64, ffn=96,
                  prefix=0, graph="dag", reveal=(1, 2), layers=3, seed=32, weight_std=0.1),
]


def _params(w):
    for l in range(w.cfg.layers):
        pk, pv = w.prefix_kv(l)
        yield w.weights[l], pk, pv


def _bf16_torch(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.bfloat16).to(
        torch.float64).numpy()


def test_round_to_bf16_matches_torch_on_fp32():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    # exact ties (a bf16 value with the half-ulp bit set), normal range only
    ties = (np.arange(0x0080, 0x0080 + 5000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.float32([0.0, 1.0, -2.5, 65504.0])])
    np.testing.assert_array_equal(round_to_bf16(x), _bf16_torch(x.astype(np.float32)))


def test_round_to_bf16_nearest_on_float64():
    rng = np.random.default_rng(4)
    x = rng.standard_normal(20000) * np.exp(rng.uniform(-5, 5, 20000))
    got = round_to_bf16(x)
    for v, g in zip(x[:2000], got[:2000]):
        # brute force: the two bf16 values that bracket |v|, nearest wins, ties to even
        a = abs(v)
        lo_bits = np.float32(a).view(np.uint32) >> 16
        cands = []
        for b in (int(lo_bits) - 1, int(lo_bits), int(lo_bits) + 1):
            c = float(np.uint32(b << 16).view(np.float32))
            cands.append((abs(c - a), b & 1, c))
        best = min(cands)[2]
        assert g == math.copysign(best, v), (v, g, best)
    # every result is bf16-representable and within half an ulp
    g32 = got.astype(np.float32)
    assert np.all(g32.view(np.uint32) & 0xFFFF == 0)
    assert np.all(np.abs(got - x) <= np.abs(x) * 2.0 ** -8)


@pytest.mark.parametrize("cfg", STACKS, ids=lambda c: f"{c.graph}{c.seed}")
def test_dense_stack_equals_textbook_chain(cfg):
    w = make_workload(cfg)
    out = stack(_params(w), w.H, w.fold_src, -1.0, n_q=cfg.n_q, n_kv=cfg.n_kv,
                eps=cfg.rms_eps, keep_inputs=True)
    x = w.H.astype(np.float64)
    for l in range(cfg.layers):
        np.testing.assert_allclose(out["inputs"][l], x, rtol=1e-10, atol=1e-10)
        pk, pv = w.prefix_kv(l)
        x = torch_dense(w.weights[l], x, pk, pv, cfg.n_q, cfg.n_kv, cfg.rms_eps)["y"]
    np.testing.assert_allclose(out["y"], x, rtol=1e-10, atol=1e-10)
    assert out["K"] == [cfg.slots] * cfg.layers


@pytest.mark.parametrize("carry", [None, "bf16"])
@pytest.mark.parametrize("tau", [0.05, 0.3])
@pytest.mark.parametrize("cfg", STACKS, ids=lambda c: f"{c.graph}{c.seed}")
def test_folded_stack_equals_regated_substituted_chain(cfg, tau, carry):
    w = make_workload(cfg)
    out = stack(_params(w), w.H, w.fold_src, tau, n_q=cfg.n_q, n_kv=cfg.n_kv,
                eps=cfg.rms_eps, carry=carry)
    N, B = cfg.num_nodes, cfg.block
    pos = np.arange(B)[None, :].repeat(N, axis=0)
    x = w.H.astype(np.float64)
    masks = []
    for l in range(cfg.layers):
        st = fold_state(x, w.fold_src, tau)
        np.testing.assert_array_equal(out["states"][l]["recompute"], st["recompute"])
        np.testing.assert_array_equal(out["states"][l]["slot_row"], st["slot_row"])
        masks.append(st["recompute"])
        src = st["src"]
        Hs = x[src, pos]
        pk, pv = w.prefix_kv(l)
        ref = torch_dense(w.weights[l], Hs, pk, pv, cfg.n_q, cfg.n_kv, cfg.rms_eps)
        x = x + (ref["h"] - Hs) + ref["F"][src, pos]
        if carry == "bf16":
            x = _bf16_torch(x)
    # a bf16 hand-over may land one bf16 ulp apart where the float64 sums, taken in a
    # different order, straddle a rounding tie
    np.testing.assert_allclose(out["y"], x, rtol=1e-9 if carry is None else 2.0 ** -7,
                               atol=1e-9)
    if carry == "bf16":
        y32 = out["y"].astype(np.float32)
        assert np.array_equal(y32.astype(np.float64), out["y"])
        assert np.all(y32.view(np.uint32) & 0xFFFF == 0), "hand-over is not bf16"
        # a skipped intermediate rounding moves about half of all elements by one ulp
        assert np.mean(out["y"] == x) > 0.995
    # the pin only bites if the layers really decide differently
    assert any(not np.array_equal(m, masks[0]) for m in masks[1:]), \
        "precondition: the recompute set changes between layers"


@pytest.mark.parametrize("cfg", STACKS, ids=lambda c: f"{c.graph}{c.seed}")
def test_tau_inf_stack_keeps_offsets(cfg):
    w = make_workload(cfg)
    out = stack(_params(w), w.H, w.fold_src, math.inf, n_q=cfg.n_q, n_kv=cfg.n_kv,
                eps=cfg.rms_eps)
    H = w.H.astype(np.float64)
    want = out["y"][0][None] + (H - H[0][None])
    np.testing.assert_allclose(out["y"], want, rtol=0, atol=1e-12)
    assert out["K"] == [cfg.block] * cfg.layers


def test_stack_rejects_unknown_carry():
    w = make_workload(STACKS[0])
    with pytest.raises(ValueError):
        stack(_params(w), w.H, w.fold_src, 0.1, n_q=2, n_kv=1, carry="fp8")
