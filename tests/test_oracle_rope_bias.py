"""Pins of the oracle's rotary-embedding and QKV-bias variant (a model family with both,
like the 7B-shaped one, uses them in every layer).

* The dense layer equals a textbook layer built from torch CPU routines, with the bias in
  the projection and the rotation written independently, as complex multiplication.
* rope() preserves norms, is the identity at position 0, and turns dot products into
  functions of the position difference only.
* With zero Q/K/V weights and no prefix, every query, key and value is the bias, so each
  head's attention output is its value bias: h = H + b_v W_o^T exactly.
* At tau = inf the closed form y_child = y_root + (H_child - H_root) still holds."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from oracle import layer, rope
from synth import custom_config, make_workload


def _cfgs():
    return [
        custom_config(name="rope-bias-a", num_nodes=5, block=6, hidden=64, n_q=2, n_kv=1,
                      head_dim=64, ffn=96, prefix=11, graph="tree3", reveal=(1, 2), seed=71,
                      rope_theta=10000.0, qkv_bias=True),
        custom_config(name="rope-bias-b", num_nodes=7, block=5, hidden=128, n_q=4, n_kv=2,
                      head_dim=64, ffn=64, prefix=0, graph="dag", reveal=(1, 2), seed=72,
                      rope_theta=1.0e6, qkv_bias=True),
    ]


def _run(w, tau, **kw):
    cfg = w.cfg
    pk, pv = w.prefix_kv(0)
    return layer(w.weights[0], w.H, w.fold_src, tau, pk, pv, n_q=cfg.n_q, n_kv=cfg.n_kv,
                 eps=cfg.rms_eps, rope_theta=cfg.rope_theta, **kw)


def _torch_rope(x, pos, theta):
    """x [N, heads, B, dh], pos [B]: pairs (x_j, x_{j+dh/2}) as complex numbers turned by
    exp(i * pos * theta^(-2j/dh))."""
    half = x.shape[-1] // 2
    inv = theta ** (-2.0 * torch.arange(half, dtype=torch.float64) / x.shape[-1])
    ang = torch.as_tensor(pos, dtype=torch.float64)[:, None] * inv[None, :]
    z = torch.complex(x[..., :half], x[..., half:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


def torch_dense_rope_bias(weights, H, pk, pv, n_q, n_kv, eps, theta):
    N, B, d = H.shape
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    x = t(H)
    wqkv = t(weights["w_qkv"])
    dh = wqkv.shape[0] // (n_q + 2 * n_kv)
    a = Fn.rms_norm(x, (d,), weight=t(weights["rms1"]), eps=eps)
    qkv = Fn.linear(a, wqkv, bias=t(weights["b_qkv"]))
    q = qkv[..., : n_q * dh].reshape(N, B, n_q, dh).transpose(1, 2)
    k = qkv[..., n_q * dh:(n_q + n_kv) * dh].reshape(N, B, n_kv, dh).transpose(1, 2)
    v = qkv[..., (n_q + n_kv) * dh:].reshape(N, B, n_kv, dh).transpose(1, 2)
    P = pk.shape[0]
    pos = np.arange(P, P + B)
    q, k = _torch_rope(q, pos, theta), _torch_rope(k, pos, theta)
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
    return dict(o=o.numpy(), h=h.numpy(), y=(h + F).numpy())


@pytest.mark.parametrize("cfg", _cfgs(), ids=lambda c: c.name)
def test_dense_equals_textbook_with_rope_and_bias(cfg):
    w = make_workload(cfg)
    assert "b_qkv" in w.weights[0]
    out = _run(w, -1.0)
    pk, pv = w.prefix_kv(0)
    ref = torch_dense_rope_bias(w.weights[0], w.H, pk, pv, cfg.n_q, cfg.n_kv, cfg.rms_eps,
                                cfg.rope_theta)
    for key in ("o", "h", "y"):
        np.testing.assert_allclose(out[key], ref[key], rtol=1e-10, atol=1e-10)
    # and the variant really changes the layer
    plain = layer({k: v for k, v in w.weights[0].items() if k != "b_qkv"}, w.H, w.fold_src,
                  -1.0, pk, pv, n_q=cfg.n_q, n_kv=cfg.n_kv, eps=cfg.rms_eps)
    assert np.max(np.abs(plain["y"] - out["y"])) > 1e-3


def test_rope_properties():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((6, 2, 64))
    k = rng.standard_normal((6, 2, 64))
    pos_q = np.array([0, 1, 5, 17, 300, 4095])
    for theta in (10000.0, 1.0e6):
        rq = rope(q, pos_q, theta)
        np.testing.assert_allclose(np.linalg.norm(rq, axis=-1), np.linalg.norm(q, axis=-1),
                                   rtol=1e-13)
        np.testing.assert_allclose(rope(q[:1], np.array([0]), theta), q[:1], rtol=0, atol=0)
        # <R(m) q, R(n) k> depends on m - n only
        for m, n in ((5, 2), (300, 17)):
            a = np.sum(rope(q[:1], np.array([m]), theta) * rope(k[:1], np.array([n]), theta))
            b = np.sum(rope(q[:1], np.array([m + 1000]), theta)
                       * rope(k[:1], np.array([n + 1000]), theta))
            assert abs(a - b) <= 1e-9 * max(1.0, abs(a))


def test_bias_alone_closed_form():
    cfg = _cfgs()[1]                          # no prefix
    w = make_workload(cfg)
    wt = dict(w.weights[0])
    wt["w_qkv"] = np.zeros_like(wt["w_qkv"])
    out = layer(wt, w.H, w.fold_src, 0.05, w.prefix_kv(0)[0], w.prefix_kv(0)[1], n_q=cfg.n_q,
                n_kv=cfg.n_kv, eps=cfg.rms_eps, rope_theta=cfg.rope_theta)
    dh, g = cfg.head_dim, cfg.n_q // cfg.n_kv
    bv = wt["b_qkv"][(cfg.n_q + cfg.n_kv) * dh:].astype(np.float64).reshape(cfg.n_kv, dh)
    o_want = np.concatenate([bv[h // g] for h in range(cfg.n_q)])
    np.testing.assert_allclose(out["o"], np.broadcast_to(o_want, out["o"].shape), rtol=0,
                               atol=1e-12)
    h_want = w.H.astype(np.float64) + o_want @ wt["w_o"].astype(np.float64).T
    np.testing.assert_allclose(out["h"], h_want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("cfg", _cfgs(), ids=lambda c: c.name)
def test_tau_inf_closed_form_with_rope_and_bias(cfg):
    w = make_workload(cfg)
    out = _run(w, math.inf)
    H = w.H.astype(np.float64)
    np.testing.assert_allclose(out["y"], out["y"][0][None] + (H - H[0][None]), rtol=0,
                               atol=1e-12)
