"""Pins of the oracle's layer arithmetic (CPU only).

  * tau < 0 (nothing folds) equals a textbook dense pre-norm GQA layer assembled from
    torch CPU library routines (rms_norm, linear, scaled_dot_product_attention, silu);
  * at any tau the folded layer equals that textbook layer run on a substituted input
    (each folded row replaced by its resolved source row), recombined as the method
    prescribes: own residual stream + corrected attention projected by W_o + the
    source's FFN output;
  * tau = +inf has the closed form y_child = y_root + (H_child - H_root);
  * tau = 0 equals the dense layer when no child row equals its source;
  * serialised branch-by-branch execution equals the packed batched execution;
  * evaluating a subset of slots gives the same values as the full evaluation;
  * the online-softmax merge of prefix partials and block keys (used by the kernels)
    equals one softmax over the concatenated keys."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import fold_state, layer, serial_layer
from parity_util import random_case
from synth import CONFIGS, custom_config, make_workload


def torch_dense(weights, H, pk, pv, n_q, n_kv, eps):
    """Textbook dense layer on every slot (float64, torch CPU library routines)."""
    N, B, d = H.shape
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    x = t(H)
    wqkv = t(weights["w_qkv"])
    dh = wqkv.shape[0] // (n_q + 2 * n_kv)
    a = Fn.rms_norm(x, (d,), weight=t(weights["rms1"]), eps=eps)
    qkv = Fn.linear(a, wqkv)
    q = qkv[..., : n_q * dh].reshape(N, B, n_q, dh).transpose(1, 2)
    k = qkv[..., n_q * dh:(n_q + n_kv) * dh].reshape(N, B, n_kv, dh).transpose(1, 2)
    v = qkv[..., (n_q + n_kv) * dh:].reshape(N, B, n_kv, dh).transpose(1, 2)
    P = pk.shape[0]
    kp = t(pk).transpose(0, 1).unsqueeze(0).expand(N, n_kv, P, dh)
    vp = t(pv).transpose(0, 1).unsqueeze(0).expand(N, n_kv, P, dh)
    keys = torch.cat([kp, k], dim=2).contiguous()
    vals = torch.cat([vp, v], dim=2).contiguous()
    o = Fn.scaled_dot_product_attention(q.contiguous(), keys, vals, enable_gqa=True)
    o = o.transpose(1, 2).reshape(N, B, n_q * dh)
    h = x + Fn.linear(o, t(weights["w_o"]))
    a2 = Fn.rms_norm(h, (d,), weight=t(weights["rms2"]), eps=eps)
    ff = weights["w_down"].shape[1]
    wgu = t(weights["w_gate_up"])
    F = Fn.linear(Fn.silu(Fn.linear(a2, wgu[:ff])) * Fn.linear(a2, wgu[ff:]), t(weights["w_down"]))
    return dict(o=o.numpy(), h=h.numpy(), F=F.numpy(), y=(h + F).numpy())


def _run(w, tau, **kw):
    cfg = w.cfg
    pk, pv = w.prefix_kv(0)
    return layer(w.weights[0], w.H, w.fold_src, tau, pk, pv, n_q=cfg.n_q, n_kv=cfg.n_kv,
                 eps=cfg.rms_eps, **kw)


SMALL = [
    custom_config(),
    custom_config(num_nodes=7, block=5, hidden=64, n_q=4, n_kv=2, head_dim=64, ffn=96,
                  prefix=0, graph="dag", reveal=(1, 2), seed=21),
    custom_config(num_nodes=6, block=12, hidden=128, n_q=6, n_kv=2, head_dim=64, ffn=64,
                  prefix=37, graph="chain", reveal=(1, 3), ripple_len=5.0, seed=5),
]


# Every fourth seeded random shape of the GPU parity sweep (GQA groups, head_dim 128,
# prefixes up to 2100 keys, blocks up to 80, up to 24 nodes), without rotary embedding and
# bias, which the textbook layer here does not have.
RANDOM = [random_case(s)[0] for s in range(0, 32, 4)]
RANDOM = [c.with_(name=c.name.replace("-rope", "").replace("-bias", ""), rope_theta=0.0,
                  qkv_bias=False) for c in RANDOM]


@pytest.mark.parametrize("cfg", SMALL + [CONFIGS[0]] + RANDOM, ids=lambda c: c.name + str(c.seed))
def test_dense_equals_textbook_layer(cfg):
    w = make_workload(cfg)
    out = _run(w, -1.0)
    pk, pv = w.prefix_kv(0)
    ref = torch_dense(w.weights[0], w.H, pk, pv, cfg.n_q, cfg.n_kv, cfg.rms_eps)
    assert out["K"] == cfg.slots
    for key in ("o", "h", "y"):
        np.testing.assert_allclose(out[key], ref[key], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(out["F"], ref["F"].reshape(cfg.slots, -1), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("tau", [0.02, 0.05, 0.2, 1.0])
@pytest.mark.parametrize("cfg", SMALL + [CONFIGS[0]] + RANDOM, ids=lambda c: c.name + str(c.seed))
def test_folded_equals_textbook_on_substituted_input(cfg, tau):
    w = make_workload(cfg)
    out = _run(w, tau)
    N, B = cfg.num_nodes, cfg.block
    src = out["src"]
    pos = np.arange(B)[None, :].repeat(N, axis=0)
    Hs = w.H[src, pos]                                   # each row -> its resolved source row
    pk, pv = w.prefix_kv(0)
    ref = torch_dense(w.weights[0], Hs, pk, pv, cfg.n_q, cfg.n_kv, cfg.rms_eps)
    want = (w.H.astype(np.float64) + (ref["h"] - Hs.astype(np.float64))
            + ref["F"][src, pos])
    np.testing.assert_allclose(out["o"], ref["o"], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(out["y"], want, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("cfg", SMALL + [CONFIGS[0]], ids=lambda c: c.name + str(c.seed))
def test_tau_inf_closed_form(cfg):
    w = make_workload(cfg)
    out = _run(w, math.inf)
    H = w.H.astype(np.float64)
    want = out["y"][0][None] + (H - H[0][None])
    np.testing.assert_allclose(out["y"], want, rtol=0, atol=1e-12)
    out32 = _run(w, math.inf, dtype=np.float32)
    np.testing.assert_allclose(out32["y"], want, rtol=0, atol=1e-5 * np.abs(want).max())


@pytest.mark.parametrize("cfg", [CONFIGS[0], SMALL[2]], ids=lambda c: c.name)
def test_tau_zero_equals_dense(cfg):
    w = make_workload(cfg)
    st = fold_state(w.H, w.fold_src, 0.0)
    assert not np.any(st["r32"][1:] == 0), "precondition: no child row equals its source"
    np.testing.assert_array_equal(_run(w, 0.0)["y"], _run(w, -1.0)["y"])


@pytest.mark.parametrize("tau", [0.05, 0.3])
@pytest.mark.parametrize("cfg", SMALL + [CONFIGS[0]], ids=lambda c: c.name + str(c.seed))
def test_serial_equals_batched(cfg, tau):
    w = make_workload(cfg)
    pk, pv = w.prefix_kv(0)
    ys = serial_layer(w.weights[0], w.H, w.fold_src, tau, pk, pv, n_q=cfg.n_q, n_kv=cfg.n_kv,
                      eps=cfg.rms_eps)
    np.testing.assert_allclose(ys, _run(w, tau)["y"], rtol=1e-12, atol=1e-12)


def test_slot_subset_matches_full():
    w = make_workload(SMALL[2])
    full = _run(w, 0.05)
    picks = [(0, 0), (5, 11), (3, 4), (4, 4), (2, 7)]
    sub = _run(w, 0.05, slots=picks)
    for (n, i) in picks:
        # same arithmetic; only the BLAS blocking of the row subset may differ
        np.testing.assert_allclose(sub["y"][n, i], full["y"][n, i], rtol=1e-13, atol=1e-13)
    assert np.isnan(sub["y"][1, 1]).all()


def test_fold_state_injection_is_used():
    w = make_workload(SMALL[0])
    dense = fold_state(w.H, w.fold_src, -1.0)
    np.testing.assert_array_equal(_run(w, 0.5, state=dense)["y"], _run(w, -1.0)["y"])


def test_online_softmax_merge_identity():
    """The kernels split the keys into prefix chunks and the block, keep (max, sum,
    normalised output) per chunk in base 2, and merge; the result must equal one softmax
    over all keys."""
    rng = np.random.default_rng(0)
    dh, P, B = 32, 70, 9
    q = rng.standard_normal(dh)
    keys = rng.standard_normal((P + B, dh)) * 2
    vals = rng.standard_normal((P + B, dh))
    s = keys @ q / math.sqrt(dh)
    w = np.exp(s - s.max())
    ref = (w / w.sum()) @ vals
    s2 = s * math.log2(math.e)
    chunks = [(0, 32), (32, 64), (64, 70)]
    lse, outs = [], []
    for a, b in chunks:
        m = s2[a:b].max()
        l = np.sum(2.0 ** (s2[a:b] - m))
        outs.append((2.0 ** (s2[a:b] - m)) @ vals[a:b] / l)
        lse.append(m + math.log2(l))
    M = max(max(lse), s2[P:].max())
    L = sum(2.0 ** (x - M) for x in lse) + np.sum(2.0 ** (s2[P:] - M))
    O = sum(2.0 ** (x - M) * o for x, o in zip(lse, outs)) + (2.0 ** (s2[P:] - M)) @ vals[P:]
    np.testing.assert_allclose(O / L, ref, rtol=1e-12, atol=1e-13)


def _layer_of(cfg, w, tau, attn, state=None):
    pk, pv = w.prefix_kv(0)
    return layer(w.weights[0], w.H, w.fold_src, tau, pk, pv, n_q=cfg.n_q, n_kv=cfg.n_kv,
                 eps=cfg.rms_eps, attn=attn, state=state)


def test_reuse_mode_closed_form_and_limits():
    """REUSE variant: a folded slot takes its resolved source's attention output, so its
    output differs from the source's by exactly its own input delta; with nothing folded
    (tau < 0) and with everything folded onto the root (tau = inf, where every branch's
    block keys are the root's rows) it equals the corrected layer; in between it does not."""
    cfg = custom_config(name="reuse", num_nodes=7, block=6, hidden=64, n_q=4, n_kv=2,
                        head_dim=64, ffn=128, prefix=9, graph="dag", reveal=(1, 2), seed=51)
    w = make_workload(cfg)
    st = fold_state(w.H, w.fold_src, 0.3)
    assert 0 < int((~st["recompute"]).sum())
    r = _layer_of(cfg, w, 0.3, "reuse", state=st)
    src = st["src"]
    for n in range(cfg.num_nodes):
        for i in range(cfg.block):
            m = src[n, i]
            if m != n:
                delta = w.H[n, i].astype(np.float64) - w.H[m, i].astype(np.float64)
                np.testing.assert_allclose(r["y"][n, i] - r["y"][m, i], delta, rtol=0,
                                           atol=1e-12)
    c = _layer_of(cfg, w, 0.3, "correct", state=st)
    assert np.max(np.abs(r["y"] - c["y"])) > 1e-6          # the correction matters here
    for tau in (-1.0, math.inf):
        a = _layer_of(cfg, w, tau, "reuse")
        b = _layer_of(cfg, w, tau, "correct")
        np.testing.assert_allclose(a["y"], b["y"], rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        _layer_of(cfg, w, 0.3, "other")


@pytest.mark.parametrize("cid", [0, 1, 2])
def test_attention_output_check_sees_the_correction(cid):
    """Guard for the GPU parity tests.  On the benchmark workloads the layer output y
    alone cannot tell the corrected attention of a folded slot (its own branch's block
    keys and values, [SF] implementation memo) from the source's reused one: the residual
    stream H dominates y, and the two modes differ in y by less than the bf16/fp32 output
    tolerance at 7B and 3B shapes.  The attention output o itself separates them by far
    more than that tolerance, so a kernel that skipped the correction fails the GPU
    tests' per-tensor check of o (and of h at the 7B shape)."""
    cfg = CONFIGS[cid]
    w = make_workload(cfg)
    st = fold_state(w.H, w.fold_src, cfg.tau)
    assert int((~st["recompute"]).sum()) > 0
    a = _layer_of(cfg, w, cfg.tau, "correct", state=st)
    b = _layer_of(cfg, w, cfg.tau, "reuse", state=st)
    tol = {"f32": 1e-3, "bf16": 2e-2}[cfg.dtype]

    def mar(x, ref):
        return float(np.max(np.abs(x - ref)) / np.max(np.abs(ref)))

    d_o = mar(b["o"], a["o"])
    assert d_o > 4 * tol, (cfg.name, d_o)
    # packed rows keep their own attention in both modes, so only folded slots differ
    rec = st["recompute"]
    np.testing.assert_array_equal(a["o"][rec], b["o"][rec])
