"""GPU parity of the LM head + per-branch argmax (specfold_lm_head_argmax, called through
the C ABI) against the oracle's lm_head_argmax.

The kernels normalise each packed row into the model dtype before the product (bf16 rows
for bf16 models) and accumulate in fp32.  Rounding a_kj to the dtype moves it by at most
half an ulp, u |a_kj| (u = 2^-9 for bf16, 2^-24 for fp32), independently per element, so
the logit moves by a sum of independent terms of standard deviation <= u |a_kj w_vj| /
sqrt(3); six standard deviations of that sum, 6 u sqrt(sum_j (a_kj w_vj)^2), plus 2^-20
sum_j |a_kj w_vj| for the fp32 accumulation, give the tolerance e(k, v).  (The worst case
u sum_j |a_kj w_vj|, all errors aligned, is about 0.18 at the 7B shape, wider than the
usual gap between the two largest of 152064 logits.)  Checks per evaluated packed row k,
with t the oracle's token and g the kernel's:
  * g == t wherever the oracle's top-1 / top-2 margin exceeds 2 * max_v e(k, v);
  * always: logit[k, g] >= logit[k, t] - (e(k, g) + e(k, t))  (g is a maximum within the
    error), and |row_logit_gpu[k] - logit[k, g]| <= e(k, g);
  * token[n, i] == row_token_gpu[slot_row[n, i]] exactly (the gather).
The fold state comes from the oracle (its masks, provenance and packing are the ones the
layer's kernels reproduce bit-exactly)."""
import numpy as np
import pytest
import torch

from oracle import fold_state, lm_head_argmax
from synth import CONFIGS, VOCAB_7B, custom_config, lm_head_weights, make_workload

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from branch_folding_amd import _lib as L
    L.lib()
    return L


def _to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(dtype).cuda()


def _gpu_lm_head(cfg, H, st, g, w, vocab):
    """specfold_lm_head_argmax on hidden rows H with fold state st: (row_token, row_logit,
    token) on the host."""
    L = _dev()
    from branch_folding_amd.runner import shape_of
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    S, K = cfg.slots, st["K"]
    sh = shape_of(cfg)
    ws_bytes = L.specfold_lm_head_workspace_bytes(sh, vocab)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    hid = _to_dev(H.reshape(S, cfg.hidden), dt)
    gd, wd = _to_dev(g, dt), _to_dev(w, dt)
    ps = torch.zeros(S, dtype=torch.int32)
    ps[:K] = torch.from_numpy(st["packed_slot"].astype(np.int32))
    ps = ps.cuda()
    sr = torch.from_numpy(st["slot_row"].reshape(-1).astype(np.int32)).cuda()
    cnt = torch.tensor([K], dtype=torch.int32, device="cuda")
    rt = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    rl = torch.zeros(S, dtype=torch.float32, device="cuda")
    tok = torch.full((S,), -7, dtype=torch.int32, device="cuda")
    L.specfold_lm_head_argmax(sh, vocab, gd, wd, hid, ps, sr, cnt, rt, rl, tok, ws, ws_bytes)
    torch.cuda.synchronize()
    return rt.cpu().numpy(), rl.cpu().numpy(), tok.cpu().numpy().reshape(st["slot_row"].shape)


def _run(cfg, H, fold_src, tau, vocab, rows=None):
    print(f"[gpu] lm head {cfg.name} V={vocab} tau={tau}", flush=True)
    g, w = lm_head_weights(cfg, vocab)
    st = fold_state(H, fold_src, tau)
    S, K = cfg.slots, st["K"]
    rt, rl, tok = _gpu_lm_head(cfg, H, st, g, w, vocab)
    # the gather is exact
    np.testing.assert_array_equal(tok, rt[st["slot_row"]])
    ref = lm_head_argmax(H, g, w, st, eps=cfg.rms_eps, rows=rows)
    u = 2.0 ** -9 if cfg.dtype == "bf16" else 2.0 ** -24
    flat = H.reshape(S, cfg.hidden).astype(np.float64)
    ks = ref["rows"]
    x = flat[st["packed_slot"][ks]]
    a = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + cfg.rms_eps) * g.astype(np.float64)
    w64 = w.astype(np.float64)
    e = 6 * u * np.sqrt((a * a) @ (w64 * w64).T) + 2.0 ** -20 * (np.abs(a) @ np.abs(w64).T)
    del w64
    lg = ref["logits"]
    exact = 0
    for r, k in enumerate(ks):
        t, gg = int(ref["row_token"][k]), int(rt[k])
        assert 0 <= gg < vocab, (k, gg)
        # with one token in the vocabulary there is no runner-up: the pick is forced
        top2 = np.partition(lg[r], -2)[-2:] if vocab > 1 else np.array([-np.inf, lg[r, 0]])
        if top2[1] - top2[0] > 2 * e[r].max():
            assert gg == t, (k, gg, t)
            exact += 1
        assert lg[r, gg] >= lg[r, t] - (e[r, gg] + e[r, t]), (k, gg, t)
        assert abs(rl[k] - lg[r, gg]) <= e[r, gg] + 1e-6, (k, rl[k], lg[r, gg])
    print(f"[gpu]   K={K} rows checked {len(ks)}, {exact} outside the tie band", flush=True)
    assert exact >= len(ks) // 2
    return st


@pytest.mark.parametrize("tau", [0.05, -1.0])
def test_lm_head_small_bf16_ragged_vocab(tau):
    cfg = custom_config(name="lm-bf16", num_nodes=9, block=16, hidden=256, dtype="bf16",
                        graph="dag", reveal=(1, 2), seed=41)
    w = make_workload(cfg, weights=False)
    _run(cfg, w.H, w.fold_src, tau, vocab=1000)      # 1000 = 7 * 128 + 104 columns


def test_lm_head_small_fp32():
    cfg = custom_config(name="lm-f32", num_nodes=5, block=12, hidden=128, dtype="f32",
                        graph="chain", seed=42)
    w = make_workload(cfg, weights=False)
    _run(cfg, w.H, w.fold_src, 0.05, vocab=333)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("vocab", [1, 17, 65])
def test_lm_head_tiny_vocab(vocab, dtype):
    """Vocabularies smaller than one wave's 64 columns (one token: every pick is token 0),
    and one column past a wave."""
    cfg = custom_config(name=f"lm-tiny-{dtype}", num_nodes=4, block=9, hidden=128, dtype=dtype,
                        graph="tree3", seed=43)
    w = make_workload(cfg, weights=False)
    st = _run(cfg, w.H, w.fold_src, 0.05, vocab=vocab)
    assert st["K"] > 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lm_head_row_without_finite_logit(dtype):
    """A packed row whose hidden state is NaN has no logit above -inf: its token is -1 and
    its logit -inf (the header's contract), and every other row's token and logit equal a
    clean run's."""
    cfg = custom_config(name=f"lm-nan-{dtype}", num_nodes=4, block=9, hidden=128, dtype=dtype,
                        graph="tree3", seed=44)
    w = make_workload(cfg, weights=False)
    g, wl = lm_head_weights(cfg, 300)
    st = fold_state(w.H, w.fold_src, 0.05)
    assert st["packed_slot"][0] == 0                  # the root's first slot is packed row 0
    rt0, rl0, tok0 = _gpu_lm_head(cfg, w.H, st, g, wl, 300)
    Hn = w.H.copy()
    Hn[0, 0, :] = np.nan
    rt, rl, tok = _gpu_lm_head(cfg, Hn, st, g, wl, 300)
    K = st["K"]
    assert rt[0] == -1 and rl[0] == -np.inf
    np.testing.assert_array_equal(rt[1:K], rt0[1:K])
    np.testing.assert_array_equal(rl[1:K], rl0[1:K])
    np.testing.assert_array_equal(tok, rt[st["slot_row"]])
    assert np.all(tok[st["slot_row"] == 0] == -1)


def test_lm_head_7b_full_vocab_sampled_rows():
    """7B shape, 1 + 15 branches, the full 152064-token vocabulary, in the benchmark's
    launch configuration; the oracle evaluates 10 sampled packed rows one by one."""
    cfg = CONFIGS[1]
    w = make_workload(cfg, weights=False)
    K = fold_state(w.H, w.fold_src, cfg.tau)["K"]
    rng = np.random.default_rng(5)
    rows = sorted({0, K - 1, K // 2} | set(int(r) for r in rng.integers(0, K, 7)))
    _run(cfg, w.H, w.fold_src, cfg.tau, vocab=VOCAB_7B, rows=rows)
