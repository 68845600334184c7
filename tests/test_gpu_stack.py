"""GPU parity of the layer stack (specfold_stack_forward) against the oracle's stack.

Layer l runs on layer l-1's output.  After the first layer the GPU's inputs differ from
the oracle's by the rounding of the GPU's fp32/bf16 arithmetic (the oracle's layers run in
float64 -- float32 for the 28-layer stack, whose rounding is still far below the bf16
tolerance -- and hand bf16 models' outputs on in bf16).  If the inputs of a child row c
and of its fold source's row p carry errors e_c and e_p, then with a = ||e_c - e_p|| / ||p||
and b = ||e_p|| / ||p|| (b < 1) the ratio r = ||c - p|| / ||p|| moves by at most
(a + r b) / (1 - b), plus the fp32 rounding of the ratio itself (2e-5 (1 + r), what layer
0 shows on identical inputs).  The GPU's input of every layer is read back by running the
stack on its first l layers, so this bound is evaluated per slot from the actual input
errors.  So:
  * every layer on its own: the GPU layer entry point fed the oracle's input of layer l
    decides bit-exactly outside the tie band and matches the oracle's layer-l output to
    the layer tolerance;
  * the stack with the oracle's per-layer fold states fed in (SPECFOLD_FLAG_FOLD_STATE_IN):
    the GPU's ratios on its own inputs stay within the bound above of the oracle's, and
    the last output agrees with the oracle's to the layer tolerance times sqrt(L).  The
    per-layer rounding errors (bf16 h and y on the GPU) are independent and add up like
    a random walk over the L layers; the sqrt(L) widening is that walk's growth;
  * the stack running its own gates: every GPU ratio is within the bound of the oracle's,
    so a decision can differ only where the oracle's ratio lies within the bound of tau;
    every node whose own and whose fold-source ancestors' decisions all agree meets the
    output bound above;
  * the stack equals chaining specfold_layer_forward calls, bit for bit."""
import math

import numpy as np
import pytest
import torch

from oracle import stack
from parity_util import TOL, assert_fold_state_equal, max_abs_rel, random_case
from synth import CONFIGS, custom_config, iter_layers, make_workload

pytestmark = pytest.mark.gpu

# fp32 rounding of the GPU's ratio on identical inputs, relative to 1 + r
RATIO_ROUNDING = 2e-5


def _ratio_bound(x_gpu, x_ora, r_ora, fold_src):
    """Per slot, the largest |r_gpu - r_oracle| that the input errors e = x_gpu - x_ora
    allow: (a + r b) / (1 - b) + rounding, a = ||e_c - e_p|| / ||p||, b = ||e_p|| / ||p||
    (infinite where b >= 1 or p = 0; the root row has no ratio)."""
    x_ora = np.asarray(x_ora, dtype=np.float64)
    e = np.asarray(x_gpu, dtype=np.float64) - x_ora
    N = len(fold_src)
    out = np.full(r_ora.shape, np.inf)
    for n in range(1, N):
        p = int(fold_src[n])
        pn = np.linalg.norm(x_ora[p], axis=-1)
        with np.errstate(divide="ignore", invalid="ignore"):
            a = np.linalg.norm(e[n] - e[p], axis=-1) / pn
            b = np.linalg.norm(e[p], axis=-1) / pn
            r = r_ora[n]
            bnd = (a + r * b) / (1 - b) + RATIO_ROUNDING * (1 + r)
        out[n] = np.where((pn > 0) & (b < 1), bnd, np.inf)
    return out


def _gpu_inputs(ds, tau, state_in, nl):
    """The GPU's input of every layer: H, then the stack's output after 1, 2, ... layers
    (the same launches as the full run, so bit-identical to its hand-overs)."""
    xs = [ds.H.float().cpu().numpy().reshape(ds.cfg.num_nodes, ds.cfg.block, -1)]
    for l in range(1, nl):
        ds.forward(tau, state_in=state_in, num_layers=l)
        torch.cuda.synchronize()
        xs.append(ds.output_numpy())
    return xs


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from branch_folding_amd import _lib as L
    from branch_folding_amd import runner
    L.lib()
    return L, runner


def _say(msg):
    print(msg, flush=True)


def _oracle_and_device_stack(runner, cfg, nl, tau, oracle_dtype=np.float64):
    """Draw every layer once: upload it to a DeviceStack and feed it to the oracle's stack
    (one layer's weights on the host at a time)."""
    ds = runner.DeviceStack(cfg, (), _hidden(cfg), _graph(cfg))

    def params():
        for l, w, c in iter_layers(cfg, nl, workers=8):
            ds.add_layer(w, c)
            _say(f"[gpu]   layer {l} drawn and uploaded; oracle layer {l}")
            yield w, c[:cfg.prefix, 0], c[:cfg.prefix, 1]
    ora = stack(params(), _hidden(cfg), _graph(cfg), tau, n_q=cfg.n_q, n_kv=cfg.n_kv,
                eps=cfg.rms_eps, dtype=oracle_dtype,
                carry="bf16" if cfg.dtype == "bf16" else None, keep_inputs=True)
    return ora, ds


_WL = {}


def _base(cfg):
    if cfg not in _WL:
        _WL.clear()
        _WL[cfg] = make_workload(cfg, layers=1, weights=False)
    return _WL[cfg]


def _hidden(cfg):
    return _base(cfg).H


def _graph(cfg):
    return _base(cfg).fold_src


def _device_stack(runner, cfg, nl):
    return runner.DeviceStack(cfg, ((w, c) for _, w, c in iter_layers(cfg, nl, workers=8)),
                              _hidden(cfg), _graph(cfg))


def _gpu_states_as_input(ora_states):
    return [dict(recompute=s["recompute"], src_node=s["src"], packed_slot=s["packed_slot"],
                 slot_row=s["slot_row"], packed_count=np.array([s["K"]], np.int32))
            for s in ora_states]


def _check_stack(cfg, nl, tau, L, runner, oracle_dtype=np.float64):
    _say(f"[gpu] stack {cfg.name} layers={nl} tau={tau} S={cfg.slots}")
    ora, ds = _oracle_and_device_stack(runner, cfg, nl, tau, oracle_dtype)
    assert ds.num_layers == nl
    tol = TOL[cfg.dtype]
    tol_stack = tol * math.sqrt(nl)

    # (0) every layer on the oracle's own input of that layer
    worst = 0.0
    for l in range(nl):
        y = ds.layer_forward(l, ora["inputs"][l], tau)
        torch.cuda.synchronize()
        if not assert_fold_state_equal(ds.fold_states()[l], ora["states"][l], tau):
            _say(f"[gpu]   layer {l}: a tie-band slot decided differently; the oracle's "
                 "fold state is fed in")
            y = ds.layer_forward(l, ora["inputs"][l], tau,
                                 state_in=_gpu_states_as_input([ora["states"][l]])[0])
            torch.cuda.synchronize()
        want = ora["inputs"][l + 1] if l + 1 < nl else ora["y"]
        got = y.float().cpu().numpy().reshape(want.shape)
        err = max_abs_rel(got, want)
        worst = max(worst, err)
        _say(f"[gpu]   layer {l} alone: K={ora['K'][l]} max_abs_rel={err:.3e}")
        assert err <= tol, (l, err)
    _say(f"[gpu]   per layer: max_abs_rel <= {worst:.3e} over {nl} layers (tol {tol})")

    # (1) oracle decisions fed in: outputs and the GPU's own ratios at every layer
    ds.load_states(_gpu_states_as_input(ora["states"]))
    ds.forward(tau, state_in=True)
    torch.cuda.synchronize()
    err = max_abs_rel(ds.output_numpy(), ora["y"])
    _say(f"[gpu]   forced: max_abs_rel={err:.3e} (bound {tol_stack:.2e}) K={ora['K']}")
    assert err <= tol_stack
    fs = _graph(cfg)
    gstates = ds.fold_states()
    xs = _gpu_inputs(ds, tau, True, nl)
    worst, worst_frac = 0.0, 0.0
    for l, (g, o) in enumerate(zip(gstates, ora["states"])):
        r_o = o["r64"][1:]
        r_g = g["ratio"][1:].astype(np.float64)
        fin = np.isfinite(r_o)
        np.testing.assert_array_equal(np.isfinite(r_g), fin)
        bnd = _ratio_bound(xs[l], ora["inputs"][l], o["r64"], fs)[1:]
        d = np.abs(r_g[fin] - r_o[fin])
        if d.size:
            worst = max(worst, float(d.max()))
            worst_frac = max(worst_frac, float(np.max(d / bnd[fin])))
        assert np.all(d <= bnd[fin]), (l, float(np.max(d - bnd[fin])))
    _say(f"[gpu]   forced: ratio drift max={worst:.3e}, at most {worst_frac:.2f} of its "
         "per-slot bound")

    # (2) the GPU's own decisions.  Every GPU ratio lies within its per-slot bound of the
    # oracle's, so a decision can differ only where the oracle's ratio lies within that
    # bound of tau.  A node's outputs depend only on its own slots and those of its
    # fold-source ancestors (gate, provenance, its block keys and values, its source's FFN
    # row), so every node none of whose decisions -- nor any ancestor's -- differed at any
    # layer is compared against the oracle's output.
    ds.forward(tau)
    torch.cuda.synchronize()
    y_free = ds.output_numpy()
    gst = ds.fold_states()
    xs = _gpu_inputs(ds, tau, False, nl)
    N = cfg.num_nodes
    tainted = np.zeros(N, dtype=bool)
    for l in range(nl):
        o, g = ora["states"][l], gst[l]
        bnd = _ratio_bound(xs[l], ora["inputs"][l], o["r64"], fs)
        fin = np.isfinite(o["r64"])
        fin[0] = False
        with np.errstate(invalid="ignore"):            # inf - inf on the root's row
            d = np.abs(g["ratio"].astype(np.float64) - o["r64"])
        assert np.all(d[fin] <= bnd[fin]), (l, float(np.max(d[fin] - bnd[fin])))
        diff = g["recompute"] != o["recompute"]
        if l == 0:
            assert_fold_state_equal(g, o, tau)
        if diff.any():
            with np.errstate(invalid="ignore"):
                near = np.abs(o["r64"] - tau) <= bnd
            assert not (diff & ~near).any(), f"layer {l}: a decision differs away from tau"
            new = diff & ~tainted[:, None]
            if new.any():
                _say(f"[gpu]   layer {l}: {int(new.sum())} near-tau decisions differ at "
                     f"nodes {sorted(set(np.nonzero(new)[0].tolist()))}")
            tainted |= diff.any(axis=1)
            for n in range(1, N):                   # nodes are numbered topologically
                tainted[n] |= tainted[fs[n]]
        elif not tainted.any():
            np.testing.assert_array_equal(g["slot_row"], o["slot_row"])
            assert g["K"] == o["K"]
    keep = ~tainted
    assert keep[0]
    err = max_abs_rel(y_free[keep], ora["y"][keep])
    _say(f"[gpu]   free: {int(keep.sum())} of {N} nodes compared, max_abs_rel={err:.3e}")
    assert err <= tol_stack
    del ds
    torch.cuda.empty_cache()


# small stacks: fp32 and bf16, benchmark-strength (0.02) and stronger weights that move
# the recompute set from layer to layer, ragged blocks, no prefix, wide rows
SMALL = [
    custom_config(name="stack-f32", num_nodes=6, block=8, hidden=128, n_q=2, n_kv=1,
                  head_dim=64, ffn=256, prefix=16, graph="tree3", reveal=(1, 2), layers=4,
                  seed=41, weight_std=0.15),
    custom_config(name="stack-bf16", num_nodes=10, block=33, hidden=256, n_q=4, n_kv=2,
                  head_dim=128, ffn=384, prefix=70, dtype="bf16", graph="dag", reveal=(1, 2),
                  layers=5, seed=42, weight_std=0.06),
    custom_config(name="stack-bf16-noprefix", num_nodes=7, block=16, hidden=128, n_q=2,
                  n_kv=2, head_dim=64, ffn=128, prefix=0, dtype="bf16", graph="chain",
                  reveal=(1, 2), layers=3, seed=43),
    # rows of more than 512 16-byte chunks: combine and the next gate run as two kernels.
    # Weight std 0.02: at hidden 4224 a std of 0.06 makes attention scores reach ~40, where
    # the bf16 rounding of q and k alone moves the softmax beyond the bf16 tolerance.
    custom_config(name="stack-wide-bf16", num_nodes=4, block=8, hidden=4224, n_q=2, n_kv=1,
                  head_dim=64, ffn=256, prefix=16, dtype="bf16", graph="tree3",
                  reveal=(1, 2), layers=3, seed=44, weight_std=0.02),
]


@pytest.mark.parametrize("tau", [0.05, 0.3])
@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_stack_small(cfg, tau):
    L, runner = _dev()
    _check_stack(cfg, cfg.layers, tau, L, runner)


# Three-layer stacks on every fourth seeded random layer shape (rotary embedding and bias
# off: the oracle's stack runs plain layers), mostly at thresholds where some slots fold
# and others recompute in every layer.
_STACK_TAUS = (0.05, 0.3, 0.02, 0.1, -1.0, math.inf, 0.05, 0.0)
RANDOM_STACK = [
    (c.with_(name=c.name.replace("-rope", "").replace("-bias", "") + "-x3", layers=3,
             rope_theta=0.0, qkv_bias=False), _STACK_TAUS[i])
    for i, (c, _) in enumerate(random_case(s) for s in range(1, 32, 4))]


@pytest.mark.parametrize("case", RANDOM_STACK, ids=lambda c: f"{c[0].name}-tau{c[1]}")
def test_stack_random_shapes(case):
    cfg, tau = case
    L, runner = _dev()
    _check_stack(cfg, cfg.layers, tau, L, runner)


@pytest.mark.parametrize("nl", [1, 2, 3])
def test_stack_equals_chained_layer_calls(nl):
    L, runner = _dev()
    cfg = SMALL[1]
    _say(f"[gpu] stack vs chained layers {cfg.name} layers={nl}")
    ds = _device_stack(runner, cfg, nl)
    ds.forward(0.05)
    layers = list(iter_layers(cfg, nl))
    x = runner.to_device(_hidden(cfg).reshape(cfg.slots, cfg.hidden), ds.dt, ds.device)
    got = ds.fold_states()
    for l, w, c in layers:
        dl = runner.DeviceLayer(cfg, w, c, _hidden(cfg), _graph(cfg))
        dl.set_hidden(x)
        x = dl.forward(0.05).clone()
        torch.cuda.synchronize()
        st = dl.fold_state()
        np.testing.assert_array_equal(st["recompute"], got[l]["recompute"])
        np.testing.assert_array_equal(st["slot_row"], got[l]["slot_row"])
    torch.cuda.synchronize()
    assert torch.equal(ds.out, x)
    assert not torch.equal(ds.out, ds.H)


def test_stack_graph_replay():
    """The stack captured as one HIP graph and replayed three times, with eager work and
    synchronisations between the replays (the outputs and fold states are overwritten with
    junk first): every replay equals the eager run bit for bit, fold states included."""
    L, runner = _dev()
    cfg = SMALL[1]
    nl = 3
    _say(f"[gpu] stack graph replay {cfg.name} layers={nl}")
    ds = _device_stack(runner, cfg, nl)
    ds.forward(0.05)
    torch.cuda.synchronize()
    ref = ds.out.clone()
    ref_states = ds.fold_states()
    g = ds.capture(0.05)
    torch.cuda.synchronize()
    for rep in range(3):
        ds.out.fill_(7.0)
        for st in ds.states:
            for v in st.values():
                v.fill_(3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ds.out, ref), rep
        for a, b in zip(ds.fold_states(), ref_states):
            for k in ("recompute", "src", "packed_slot", "slot_row", "K"):
                np.testing.assert_array_equal(a[k], b[k])
            np.testing.assert_array_equal(a["ratio"], b["ratio"])


def test_stack_7b_shape_two_layers():
    """The 28-layer stack's shape (7B layer, 1+31 branches, prefix 4096) on its first
    two layers; the full depth runs in test_stack_7b_full_depth."""
    L, runner = _dev()
    cfg = CONFIGS[3]
    _check_stack(cfg, 2, cfg.tau, L, runner)


@pytest.mark.timeout(1200)
def test_stack_7b_full_depth():
    """All 28 layers of the 7B-shaped stack (1+31 branches, prefix 4096, tau = 0.05) in
    the benchmark's launch configuration.  The oracle runs its layers in float32 here
    (about a second per layer on the host) rather than float64; its rounding stays four
    orders of magnitude below the bf16 tolerance."""
    L, runner = _dev()
    cfg = CONFIGS[3]
    _check_stack(cfg, cfg.layers, cfg.tau, L, runner, oracle_dtype=np.float32)
