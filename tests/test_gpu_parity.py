"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Gate masks, provenance and packing must match bit for bit (slots whose ratio lies within
1e-4 relative of tau are excluded from the mask comparison); layer outputs must agree to
max|y - y_ref| / max|y_ref| <= 1e-3 (fp32) or 2e-2 (bf16).  When a tie-band slot decides
differently, the layer is also compared with the oracle's own fold state fed to the GPU
(SPECFOLD_FLAG_FOLD_STATE_IN), so the oracle never consumes a GPU result."""
import math

import numpy as np
import pytest
import torch

from parity_util import (TOL, assert_fold_state_equal, max_abs_rel, oracle_layer,
                         oracle_state, random_case)
from synth import CONFIGS, budget_config, custom_config, make_workload

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from branch_folding_amd import _lib as L
    from branch_folding_amd.runner import DeviceLayer
    L.lib()
    return L, DeviceLayer


def _say(msg):
    print(msg, flush=True)


_WL = {}


def _workload(cfg, **kw):
    key = (cfg, tuple(sorted(kw.items())))
    if key not in _WL:
        _WL.clear()
        _WL[key] = make_workload(cfg, **kw)
    return _WL[key]


# Small and edge-case shapes: ragged blocks (B not a multiple of 16, B > 64 so the block
# phase spans two key tiles), ragged and empty prefixes, root-only graphs, MHA (g = 1),
# GQA 7:1, head_dim 64/128, deep chains and DAGs.
EDGE = [
    custom_config(name="edge-root-only", num_nodes=1, block=7, hidden=128, n_q=2, n_kv=1,
                  head_dim=64, ffn=128, prefix=5, dtype="f32", seed=31),
    custom_config(name="edge-noprefix-mha", num_nodes=5, block=13, hidden=128, n_q=2, n_kv=2,
                  head_dim=64, ffn=256, prefix=0, dtype="f32", graph="dag", reveal=(1, 2),
                  seed=32),
    custom_config(name="edge-ragged-bf16", num_nodes=9, block=70, hidden=256, n_q=7, n_kv=1,
                  head_dim=128, ffn=384, prefix=100, dtype="bf16", graph="dag_deep",
                  max_depth=6, reveal=(1, 4), seed=33),
    custom_config(name="edge-chain-bf16", num_nodes=12, block=33, hidden=384, n_q=6, n_kv=2,
                  head_dim=64, ffn=640, prefix=300, dtype="bf16", graph="chain",
                  reveal=(1, 2), seed=34),
    custom_config(name="edge-raggedN-bf16", num_nodes=3, block=9, hidden=128, n_q=3, n_kv=1,
                  head_dim=64, ffn=128, prefix=65, dtype="bf16", graph="chain", seed=36),
    custom_config(name="edge-star-f32", num_nodes=17, block=16, hidden=256, n_q=4, n_kv=4,
                  head_dim=128, ffn=256, prefix=129, dtype="f32", graph="star",
                  reveal=(1, 1), seed=35),
    # bf16 without a prefix: the block phase alone, two key tiles (100 keys)
    custom_config(name="edge-noprefix-bf16", num_nodes=6, block=100, hidden=256, n_q=4, n_kv=2,
                  head_dim=128, ffn=256, prefix=0, dtype="bf16", graph="tree3",
                  reveal=(1, 2), seed=39),
]


# bf16 prefixes of 2048+ keys take the 256-query prefix kernel (direct-to-LDS ring,
# transposed V reads): ragged last tiles (52 keys; 1 key), head_dim 128 and 64, GQA 7:1 and
# 2:1, enough packed rows for several query tiles and splits.
LONG_PREFIX = [
    custom_config(name="longp-ragged-dh128", num_nodes=9, block=40, hidden=256, n_q=7, n_kv=1,
                  head_dim=128, ffn=256, prefix=2100, dtype="bf16", graph="dag",
                  reveal=(1, 3), seed=37),
    custom_config(name="longp-ragged-dh64", num_nodes=6, block=24, hidden=256, n_q=4, n_kv=2,
                  head_dim=64, ffn=256, prefix=2049, dtype="bf16", graph="chain",
                  reveal=(1, 2), seed=38),
]


# Prefixes up to 512 keys are streamed by the block phase itself, tile by tile ahead of the
# branch's block; longer ones below the 256-query kernel's 2048 (bf16) or any length (fp32)
# run the 64-query prefix phase with split partials: the last fused length, the first
# unfused one and a ragged mid-length prefix, in both dtypes.
MID_PREFIX = [
    custom_config(name="midp-fused-bf16", num_nodes=7, block=20, hidden=256, n_q=4, n_kv=2,
                  head_dim=128, ffn=256, prefix=512, dtype="bf16", graph="tree3",
                  reveal=(1, 2), seed=93),
    custom_config(name="midp-bf16", num_nodes=7, block=20, hidden=256, n_q=4, n_kv=2,
                  head_dim=128, ffn=256, prefix=513, dtype="bf16", graph="tree3",
                  reveal=(1, 2), seed=94),
    custom_config(name="midp-f32", num_nodes=6, block=18, hidden=128, n_q=6, n_kv=2,
                  head_dim=64, ffn=256, prefix=1500, dtype="f32", graph="dag",
                  reveal=(1, 2), seed=95),
    # bf16 block phase after a prefix phase with three key tiles (130 keys, ragged), dh 64
    custom_config(name="midp-longblock-bf16", num_nodes=5, block=130, hidden=256, n_q=4,
                  n_kv=1, head_dim=64, ffn=256, prefix=600, dtype="bf16", graph="chain",
                  reveal=(1, 2), seed=96),
]


# 2048+ slots: the split-K GEMMs run 256-row tiles (8 waves); every slot compared, with
# dense (2048 packed rows = 8 row tiles) and folded (a ragged last row tile) packings.
TALL = [
    custom_config(name="tall-bf16", num_nodes=64, block=32, hidden=256, n_q=4, n_kv=2,
                  head_dim=64, ffn=512, prefix=100, dtype="bf16", graph="tree3",
                  reveal=(1, 2), seed=61),
    custom_config(name="tall-f32", num_nodes=32, block=72, hidden=128, n_q=2, n_kv=1,
                  head_dim=64, ffn=256, prefix=33, dtype="f32", graph="dag", reveal=(1, 3),
                  seed=62),
]


# Rows longer than the gate's register-held part (512 16-byte chunks: hidden > 2048 in fp32,
# > 4096 in bf16): the gate's tail loop for the ratio sums and the normalised rows.
WIDE = [
    custom_config(name="wide-f32", num_nodes=4, block=12, hidden=2304, n_q=2, n_kv=1,
                  head_dim=64, ffn=256, prefix=20, dtype="f32", graph="tree3", reveal=(1, 2),
                  seed=71),
    custom_config(name="wide-bf16", num_nodes=5, block=9, hidden=4224, n_q=4, n_kv=2,
                  head_dim=64, ffn=384, prefix=33, dtype="bf16", graph="dag", reveal=(1, 2),
                  seed=72),
]


# 512 to 2047 slots: a folded call's packed row count is known only on the device, so the
# GEMMs pick their row tile there (256-row tiles from 512 packed rows, 128-row tiles and the
# SwiGLU column slabs below).  tau = 0 packs every slot (the 256-row path), 0.05 and 0.3 fewer.
AUTO = [
    custom_config(name="auto-f32", num_nodes=12, block=48, hidden=256, n_q=4, n_kv=2,
                  head_dim=64, ffn=512, prefix=40, dtype="f32", graph="dag", reveal=(1, 2),
                  seed=91),
    custom_config(name="auto-bf16", num_nodes=20, block=40, hidden=384, n_q=6, n_kv=2,
                  head_dim=64, ffn=640, prefix=70, dtype="bf16", graph="tree3",
                  reveal=(1, 2), seed=92),
]


def _check_intermediates(dl, cfg, ref, K, L, tag, attn_slots=None):
    """Every intermediate the workspace keeps, element-wise against the oracle's, each to
    the output tolerance (max-abs-rel over the entries the oracle evaluated):
      * the packed Q|K|V rows (after bias and rotary embedding, if any), first K rows;
      * the attention output o of every slot -- a folded slot's o is corrected against
        its own branch's block keys and values, which y alone cannot show (the residual
        stream dominates y);
      * h = H + o W_o^T of every slot;
      * the packed FFN output rows F.
    attn_slots: bool [N, B] restricting the o check (REUSE: the packed slots)."""
    S, tol = cfg.slots, TOL[cfg.dtype]

    def host(which, rows):
        # rows past K of a packed tensor were never written in this call
        return dl.intermediate(which)[:rows].float().cpu().numpy().astype(np.float64)

    qkv_ref = np.concatenate([ref["Q"].reshape(K, -1), ref["K_"].reshape(K, -1),
                              ref["V"].reshape(K, -1)], axis=1)
    o_ref = ref["o"].reshape(S, -1).copy()
    if attn_slots is not None:
        o_ref[~attn_slots.reshape(-1)] = np.nan
    checks = [("qkv", host(L.SPECFOLD_T_QKV, K), qkv_ref),
              ("o", host(L.SPECFOLD_T_ATTN, S), o_ref),
              ("h", host(L.SPECFOLD_T_H, S), ref["h"].reshape(S, -1)),
              ("F", host(L.SPECFOLD_T_FFN, K), ref["F"].reshape(K, -1))]
    msg = []
    for name, got, want in checks:
        rows = np.all(np.isfinite(want), axis=1)        # rows the oracle evaluated
        assert rows.any(), name
        err = max_abs_rel(got[rows], want[rows])
        msg.append(f"{name}={err:.2e}")
        assert err <= tol, (tag, name, err, tol)
    _say(f"[gpu]   {tag} intermediates " + " ".join(msg))


def _check_layer(cfg, w, tau, L, DeviceLayer, slots=None):
    _say(f"[gpu] layer {cfg.name} tau={tau} S={cfg.slots}")
    dl = DeviceLayer(cfg, w.weights[0], w.cache, w.H, w.fold_src)
    dl.forward(tau)
    torch.cuda.synchronize()
    gst = dl.fold_state()
    ost = oracle_state(w, tau)
    masks_agree = assert_fold_state_equal(gst, ost, tau)
    y_gpu = dl.output_numpy()
    tol = TOL[cfg.dtype]
    ref = oracle_layer(w, tau, state=ost, slots=slots)
    sel = np.ones(y_gpu.shape[:2], bool) if slots is None else _slot_mask(cfg, slots)
    if masks_agree:
        err = max_abs_rel(y_gpu[sel], ref["y"][sel])
        _say(f"[gpu]   K={gst['K']} max-abs-rel={err:.3e} (tol {tol})")
        assert err <= tol
        _check_intermediates(dl, cfg, ref, ost["K"], L, "own-state")
    # conditioned on the oracle's fold state
    y_in = dl.forward(tau, state_in=dict(recompute=ost["recompute"], src_node=ost["src"],
                                         packed_slot=np.pad(ost["packed_slot"],
                                                            (0, cfg.slots - ost["K"])),
                                         slot_row=ost["slot_row"],
                                         packed_count=np.array([ost["K"]])))
    torch.cuda.synchronize()
    y_in = y_in.float().cpu().numpy().reshape(y_gpu.shape)
    err = max_abs_rel(y_in[sel], ref["y"][sel])
    _say(f"[gpu]   state-in max-abs-rel={err:.3e}")
    assert err <= tol
    _check_intermediates(dl, cfg, ref, ost["K"], L, "state-in")
    return dl, gst, ost


def _slot_mask(cfg, slots):
    m = np.zeros((cfg.num_nodes, cfg.block), bool)
    for n, i in slots:
        m[n, i] = True
    return m


@pytest.mark.parametrize("cfg", EDGE + [CONFIGS[0]], ids=lambda c: c.name)
@pytest.mark.parametrize("tau", [-1.0, 0.05, 0.3, math.inf])
def test_layer_small(cfg, tau):
    L, DeviceLayer = _dev()
    w = _workload(cfg)
    _check_layer(cfg, w, tau, L, DeviceLayer)


@pytest.mark.parametrize("cfg", WIDE, ids=lambda c: c.name)
@pytest.mark.parametrize("tau", [-1.0, 0.05, 0.3, math.inf])
def test_layer_wide_rows(cfg, tau):
    L, DeviceLayer = _dev()
    _check_layer(cfg, _workload(cfg), tau, L, DeviceLayer)


@pytest.mark.parametrize("cfg", LONG_PREFIX, ids=lambda c: c.name)
@pytest.mark.parametrize("tau", [-1.0, 0.05])
def test_layer_long_prefix(cfg, tau):
    L, DeviceLayer = _dev()
    _check_layer(cfg, _workload(cfg), tau, L, DeviceLayer)


def test_fold_steps_individually():
    """specfold_gate, specfold_resolve and specfold_pack called one by one."""
    L, DeviceLayer = _dev()
    from branch_folding_amd.runner import shape_of, to_device
    for cfg in [CONFIGS[0], EDGE[2], CONFIGS[2].with_(hidden=256)]:
        w = _workload(cfg, weights=False)
        N, B, S = cfg.num_nodes, cfg.block, cfg.slots
        sh = shape_of(cfg)
        H = to_device(w.H.reshape(S, -1), torch.bfloat16 if cfg.dtype == "bf16" else torch.float32,
                      "cuda")
        fs = torch.from_numpy(w.fold_src).cuda()
        for tau in (0.0, 0.02, 0.05, 0.1, -1.0, math.inf):
            _say(f"[gpu] fold steps {cfg.name} tau={tau}")
            ratio = torch.empty(S, device="cuda")
            rec = torch.empty(S, dtype=torch.uint8, device="cuda")
            src = torch.empty(S, dtype=torch.int32, device="cuda")
            ps = torch.empty(S, dtype=torch.int32, device="cuda")
            sr = torch.empty(S, dtype=torch.int32, device="cuda")
            cnt = torch.empty(1, dtype=torch.int32, device="cuda")
            L.specfold_gate(sh, H, fs, tau, ratio, rec)
            ost = oracle_state(w, tau)
            # resolve/pack on the oracle's mask: bit-exact whatever the tie band did
            rec_o = torch.from_numpy(ost["recompute"].reshape(-1).astype(np.uint8)).cuda()
            L.specfold_resolve(sh, rec_o, fs, src)
            L.specfold_pack(sh, rec_o, src, ps, sr, cnt)
            torch.cuda.synchronize()
            K = int(cnt.item())
            assert K == ost["K"]
            np.testing.assert_array_equal(src.cpu().numpy().reshape(N, B), ost["src"])
            np.testing.assert_array_equal(ps.cpu().numpy()[:K], ost["packed_slot"])
            np.testing.assert_array_equal(sr.cpu().numpy().reshape(N, B), ost["slot_row"])
            gst = dict(ratio=ratio.cpu().numpy().reshape(N, B),
                       recompute=rec.cpu().numpy().reshape(N, B) != 0,
                       src=ost["src"], K=ost["K"], packed_slot=ost["packed_slot"],
                       slot_row=ost["slot_row"])
            assert_fold_state_equal(gst, ost, tau)


def test_pack_maximum_slots():
    """S = 16384 slots (the supported maximum) through resolve + pack."""
    L, _ = _dev()
    from branch_folding_amd.runner import shape_of
    from oracle import pack, resolve
    cfg = custom_config(num_nodes=256, block=64, hidden=128)
    rng = np.random.default_rng(5)
    fs = np.array([-1] + [int(rng.integers(0, n)) for n in range(1, 256)], dtype=np.int32)
    rec = rng.random((256, 64)) < 0.3
    rec[0] = True
    sh = shape_of(cfg)
    S = cfg.slots
    src = torch.empty(S, dtype=torch.int32, device="cuda")
    ps = torch.empty(S, dtype=torch.int32, device="cuda")
    sr = torch.empty(S, dtype=torch.int32, device="cuda")
    cnt = torch.empty(1, dtype=torch.int32, device="cuda")
    rec_d = torch.from_numpy(rec.reshape(-1).astype(np.uint8)).cuda()
    fs_d = torch.from_numpy(fs).cuda()
    _say("[gpu] pack S=16384")
    L.specfold_resolve(sh, rec_d, fs_d, src)
    L.specfold_pack(sh, rec_d, src, ps, sr, cnt)
    torch.cuda.synchronize()
    src_o = resolve(rec, fs)
    ps_o, sr_o, K = pack(rec, src_o)
    assert int(cnt.item()) == K
    np.testing.assert_array_equal(src.cpu().numpy().reshape(256, 64), src_o)
    np.testing.assert_array_equal(ps.cpu().numpy()[:K], ps_o)
    np.testing.assert_array_equal(sr.cpu().numpy().reshape(256, 64), sr_o)


@pytest.mark.parametrize("N", [1, 2, 3, 5, 16, 17, 64, 256])
def test_resolve_longest_chains(N):
    """Provenance on a chain (node n folds onto n-1) with B = 64 positions: position i
    recomputes at node n with probability i/64, so position 0 folds all the way to the root
    (a chain of N-1 links, the longest there can be) and the rest cover every shorter length.
    A second call gives one node a malformed fold source (not in [0, n)): resolve must treat
    it as computing its own row at every position, so the oracle gets that node marked for
    recompute; the pack takes that marked mask, as the gate hands it over in the layer."""
    L, _ = _dev()
    from branch_folding_amd.runner import shape_of
    from oracle import pack, resolve
    B = 64
    cfg = custom_config(num_nodes=N, block=B, hidden=128)
    sh = shape_of(cfg)
    rng = np.random.default_rng(100 + N)
    fs = np.arange(-1, N - 1, dtype=np.int32)
    rec = rng.random((N, B)) < (np.arange(B) / B)[None, :]
    rec[0] = True
    cases = [(fs, rec, rec)]
    if N >= 3:
        bad = fs.copy()
        bad[N // 2] = N // 2 if N % 2 else -7           # itself (not < n) or negative
        rec_o = rec.copy()
        rec_o[N // 2] = True
        cases.append((bad, rec, rec_o))
    for fs_dev, rec_dev, rec_oracle in cases:
        _say(f"[gpu] resolve chain N={N}")
        src = torch.empty(N * B, dtype=torch.int32, device="cuda")
        ps = torch.empty(N * B, dtype=torch.int32, device="cuda")
        sr = torch.empty(N * B, dtype=torch.int32, device="cuda")
        cnt = torch.empty(1, dtype=torch.int32, device="cuda")
        rec_d = torch.from_numpy(rec_dev.reshape(-1).astype(np.uint8)).cuda()
        L.specfold_resolve(sh, rec_d, torch.from_numpy(fs_dev).cuda(), src)
        rec_p = torch.from_numpy(rec_oracle.reshape(-1).astype(np.uint8)).cuda()
        L.specfold_pack(sh, rec_p, src, ps, sr, cnt)
        torch.cuda.synchronize()
        src_o = resolve(rec_oracle, np.arange(-1, N - 1, dtype=np.int32))
        ps_o, sr_o, K = pack(rec_oracle, src_o)
        np.testing.assert_array_equal(src.cpu().numpy().reshape(N, B), src_o)
        assert int(cnt.item()) == K
        np.testing.assert_array_equal(ps.cpu().numpy()[:K], ps_o)
        np.testing.assert_array_equal(sr.cpu().numpy().reshape(N, B), sr_o)


def test_cfg1_full_size():
    """The 7B-shaped layer (1 + 15 branches, tau = 0.05) in the benchmark's launch
    configuration, every output slot compared."""
    L, DeviceLayer = _dev()
    w = _workload(CONFIGS[1])
    dl, gst, ost = _check_layer(CONFIGS[1], w, CONFIGS[1].tau, L, DeviceLayer)
    # determinism: a second run is bit-identical
    y1 = dl.forward(CONFIGS[1].tau).clone()
    y2 = dl.forward(CONFIGS[1].tau).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("tau", [0.0, 0.02, 0.05, 0.1])
def test_cfg2_dag_tau_sweep(tau):
    L, DeviceLayer = _dev()
    _check_layer(CONFIGS[2], _workload(CONFIGS[2]), tau, L, DeviceLayer)


def test_cfg4_stress_sampled():
    """Stress layer (1 + 63 DAG, prefix 16384, block 64) at full size; outputs compared on
    sampled slots that the oracle evaluates one by one (roots, deep fold chains, the last
    slot)."""
    L, DeviceLayer = _dev()
    cfg = CONFIGS[4]
    w = _workload(cfg)
    rng = np.random.default_rng(0)
    slots = [(0, 0), (0, cfg.block - 1), (cfg.num_nodes - 1, cfg.block - 1), (6, 5), (5, 40)]
    slots += [(int(rng.integers(0, cfg.num_nodes)), int(rng.integers(0, cfg.block)))
              for _ in range(27)]
    _check_layer(cfg, w, cfg.tau, L, DeviceLayer, slots=slots)


@pytest.mark.parametrize("n,tau", [(4, 0.05), (4, -1.0), (64, 0.05), (64, -1.0)])
def test_budget_sweep_ends(n, tau):
    """The draft-budget sweep's smallest and largest layers (7B shape, 1 + 3 and 1 + 63
    branches of the 3-ary tree), folded and dense, in the benchmark's launch configuration.
    1 + 3 compares every slot; 1 + 63 (2048 slots) compares sampled slots the oracle
    evaluates one by one: roots, the deepest leaves, the last slot."""
    L, DeviceLayer = _dev()
    cfg = budget_config(n)
    w = _workload(cfg)
    slots = None
    if cfg.slots > 512:
        rng = np.random.default_rng(1)
        slots = [(0, 0), (0, cfg.block - 1), (n - 1, cfg.block - 1), (n // 2, 3)]
        slots += [(int(rng.integers(0, n)), int(rng.integers(0, cfg.block)))
                  for _ in range(20)]
    _check_layer(cfg, w, tau, L, DeviceLayer, slots=slots)


@pytest.mark.parametrize("cfg,tau", [(EDGE[2], 0.3), (EDGE[5], 0.05), (CONFIGS[0], 0.05),
                                     (CONFIGS[1], 0.05), (AUTO[1], 0.0), (AUTO[0], 0.3)],
                         ids=["ragged-bf16-dag", "star-f32", "tiny-f32", "7b-layer",
                              "device-tile-bf16-tau0", "device-tile-f32"])
def test_layer_reuse_attention(cfg, tau):
    """REUSE variant (SPECFOLD_FLAG_REUSE_ATTENTION): a folded slot takes its resolved
    source's attention output; the O projection runs on the packed rows only.  Compared
    with the oracle's attn="reuse" layer, and on the GPU output itself the closed form
    y[n,i] - y[src,i] = H[n,i] - H[src,i] within the output tolerance."""
    _check_reuse(cfg, tau, expect_difference=True)


def _check_reuse(cfg, tau, expect_difference):
    """expect_difference: the case folds slots next to recomputed keys, so the corrected
    layer must differ from the reused one somewhere (not so where every folded slot's
    branch keys are its source's own, e.g. at tau = inf)."""
    L, DeviceLayer = _dev()
    w = _workload(cfg)
    _say(f"[gpu] reuse layer {cfg.name} tau={tau}")
    dl = DeviceLayer(cfg, w.weights[0], w.cache, w.H, w.fold_src)
    dl.forward(tau, reuse=True)
    torch.cuda.synchronize()
    gst = dl.fold_state()
    ost = oracle_state(w, tau)
    st = ost
    if not assert_fold_state_equal(gst, ost, tau):
        dl.forward(tau, reuse=True,
                   state_in=dict(recompute=ost["recompute"], src_node=ost["src"],
                                 packed_slot=np.pad(ost["packed_slot"], (0, cfg.slots - ost["K"])),
                                 slot_row=ost["slot_row"], packed_count=np.array([ost["K"]])))
        torch.cuda.synchronize()
    y = dl.output_numpy()
    ref = oracle_layer(w, tau, state=st, attn="reuse")
    tol = TOL[cfg.dtype]
    err = max_abs_rel(y, ref["y"])
    _say(f"[gpu]   K={st['K']} max-abs-rel={err:.3e} (tol {tol})")
    assert err <= tol
    # the O projection reads only the packed rows' attention output here
    _check_intermediates(dl, cfg, ref, st["K"], L, "reuse", attn_slots=st["recompute"])
    src = st["src"]
    scale = np.max(np.abs(y))
    worst = 0.0
    for n in range(cfg.num_nodes):
        for i in range(cfg.block):
            m = int(src[n, i])
            if m != n:
                d = (y[n, i] - y[m, i]) - (w.H[n, i].astype(np.float64) - w.H[m, i])
                worst = max(worst, float(np.max(np.abs(d))) / scale)
    assert worst <= tol, worst
    # the corrected and the reused layer differ once anything folds next to a recomputed key
    if expect_difference:
        dl.forward(tau)
        torch.cuda.synchronize()
        if (~st["recompute"]).any():
            assert np.max(np.abs(dl.output_numpy() - y)) > 0


@pytest.mark.parametrize("cfg", TALL, ids=lambda c: c.name)
@pytest.mark.parametrize("tau", [-1.0, 0.05])
def test_layer_tall_row_tiles(cfg, tau):
    L, DeviceLayer = _dev()
    assert cfg.slots >= 2048
    _check_layer(cfg, _workload(cfg), tau, L, DeviceLayer)


def test_layer_tall_row_tiles_reuse():
    """The REUSE variant at 2048 slots: the O projection over the packed rows with 256-row
    tiles and the split re-derived on the device by the O finish."""
    L, DeviceLayer = _dev()
    cfg = TALL[0]
    w = _workload(cfg)
    dl = DeviceLayer(cfg, w.weights[0], w.cache, w.H, w.fold_src)
    dl.forward(0.05, reuse=True)
    torch.cuda.synchronize()
    ost = oracle_state(w, 0.05)
    assert assert_fold_state_equal(dl.fold_state(), ost, 0.05)
    err = max_abs_rel(dl.output_numpy(), oracle_layer(w, 0.05, state=ost, attn="reuse")["y"])
    _say(f"[gpu] tall reuse K={ost['K']} max-abs-rel={err:.3e}")
    assert err <= TOL[cfg.dtype]


# Rotary embedding and QKV bias (model families with both): fp32 and bf16, dense and folded,
# head_dim 64 and 128, a long prefix (the 256-query prefix kernel) with rope only.
ROPE = [
    custom_config(name="rope-bias-f32", num_nodes=6, block=10, hidden=128, n_q=2, n_kv=1,
                  head_dim=64, ffn=128, prefix=21, dtype="f32", graph="dag", reveal=(1, 2),
                  seed=81, rope_theta=10000.0, qkv_bias=True),
    custom_config(name="rope-bias-bf16", num_nodes=9, block=24, hidden=256, n_q=4, n_kv=2,
                  head_dim=128, ffn=256, prefix=70, dtype="bf16", graph="tree3",
                  reveal=(1, 2), seed=82, rope_theta=1.0e6, qkv_bias=True),
    custom_config(name="rope-longp-bf16", num_nodes=6, block=24, hidden=256, n_q=4, n_kv=2,
                  head_dim=64, ffn=256, prefix=2100, dtype="bf16", graph="chain",
                  reveal=(1, 2), seed=83, rope_theta=10000.0),
]


@pytest.mark.parametrize("cfg", ROPE, ids=lambda c: c.name)
@pytest.mark.parametrize("tau", [-1.0, 0.05])
def test_layer_rope_bias(cfg, tau):
    L, DeviceLayer = _dev()
    _check_layer(cfg, _workload(cfg), tau, L, DeviceLayer)


def test_cfg1_rope_bias_full_size():
    """The 7B-shaped layer with the rotary embedding (base 10^6) and QKV bias of its model
    family, every slot compared."""
    L, DeviceLayer = _dev()
    cfg = CONFIGS[1].with_(name="7b-layer-1+15-rope-bias", rope_theta=1.0e6, qkv_bias=True)
    _check_layer(cfg, _workload(cfg), cfg.tau, L, DeviceLayer)


def _golden_gate_rows(hidden):
    """The hand-built rows of tests/golden/gate_cases.json (exact rational ratios from
    Pythagorean triples; zero-norm parents), spread over a `hidden`-wide row at columns
    that fall into different lanes and 16-byte chunks (zero columns change neither norm),
    plus rows that are not in that file: a NaN in the child, a NaN in the parent, and an
    identical pair that must fold at tau = 0.  Returns (parent rows, child rows, exact
    ratios as (num, den), den = 0 for +inf and None for NaN)."""
    import json
    import os
    spec = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "gate_cases.json")))
    cols = [0, 37, 64, hidden - 1]
    par, chi, want = [], [], []
    for case in spec["cases"]:
        p = np.zeros(hidden, np.float32)
        c = np.zeros(hidden, np.float32)
        p[cols] = case["parent"]
        c[cols] = case["child"]
        par.append(p)
        chi.append(c)
        want.append((case["r_num"], case["r_den"]))
    base = np.zeros(hidden, np.float32)
    base[cols] = [3, 4, 12, 0]                            # ||p|| = 13
    nan_c = base.copy()
    nan_c[5] = np.nan
    nan_p = base.copy()
    nan_p[70] = np.nan
    for p, c, r in ((base, nan_c, None), (nan_p, base, None), (base, base.copy(), (0, 1))):
        par.append(p)
        chi.append(c)
        want.append(r)
    return np.stack(par), np.stack(chi), want


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gate_golden_cases(dtype):
    """specfold_gate on the hand-built rows: the ratio of every finite case equals the
    exact rational to fp32 rounding, a zero-norm parent gives 0 (equal rows) or +inf, a
    NaN anywhere in either row gives NaN and recomputes, and the decision fold iff
    r <= tau holds at tau = 0 (identical rows fold), at tau equal to a case's exact
    ratio (1 and 1/2 fold), between ratios, at +inf (every finite ratio folds), below
    zero and at a NaN tau (nothing folds).  The root's rows always recompute with r = +inf."""
    L, _ = _dev()
    from branch_folding_amd.runner import shape_of
    d = 128
    par, chi, want = _golden_gate_rows(d)
    B = len(want)
    cfg = custom_config(num_nodes=2, block=B, hidden=d, dtype=dtype)
    sh = shape_of(cfg)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    H = torch.from_numpy(np.concatenate([par, chi])).to(tdt).cuda()    # every value is bf16-exact
    fs = torch.tensor([-1, 0], dtype=torch.int32, device="cuda")
    exact = np.array([np.nan if r is None else (math.inf if r[1] == 0 else r[0] / r[1])
                      for r in want])
    for tau in (1.0, 0.5, 0.0, 0.75, math.inf, -1.0, math.nan):
        _say(f"[gpu] gate golden {dtype} tau={tau}")
        ratio = torch.empty(2 * B, device="cuda")
        rec = torch.empty(2 * B, dtype=torch.uint8, device="cuda")
        L.specfold_gate(sh, H, fs, tau, ratio, rec)
        torch.cuda.synchronize()
        r = ratio.cpu().numpy().reshape(2, B)
        m = rec.cpu().numpy().reshape(2, B) != 0
        assert m[0].all() and np.isinf(r[0]).all() and (r[0] > 0).all()
        got = r[1].astype(np.float64)
        nan = np.isnan(exact)
        assert np.isnan(got[nan]).all()
        inf = np.isinf(exact)
        assert np.isinf(got[inf]).all()
        fin = ~nan & ~inf
        # the fp32 ratio of exactly representable inputs: within one fp32 rounding step
        np.testing.assert_allclose(got[fin], exact[fin], rtol=2.0 ** -23, atol=0)
        with np.errstate(invalid="ignore"):
            expect = ~(exact <= tau)
        np.testing.assert_array_equal(m[1], expect)


@pytest.mark.parametrize("cfg", AUTO, ids=lambda c: c.name)
@pytest.mark.parametrize("tau", [0.0, 0.05, 0.3])
def test_layer_device_row_tile(cfg, tau):
    """Folded layers whose GEMM row tile is chosen on the device from the packed count."""
    L, DeviceLayer = _dev()
    assert 512 <= cfg.slots < 2048
    w = _workload(cfg)
    _, gst, _ = _check_layer(cfg, w, tau, L, DeviceLayer)
    if tau == 0.0:
        assert gst["K"] >= 512            # the 256-row path ran


@pytest.mark.parametrize("cfg", MID_PREFIX, ids=lambda c: c.name)
@pytest.mark.parametrize("tau", [-1.0, 0.05])
def test_layer_mid_prefix(cfg, tau):
    L, DeviceLayer = _dev()
    _check_layer(cfg, _workload(cfg), tau, L, DeviceLayer)


# Seeded random shapes (parity_util.random_case): combinations no hand-picked case names.
RANDOM = [random_case(s) for s in range(32)]


@pytest.mark.parametrize("case", RANDOM, ids=lambda c: f"{c[0].name}-tau{c[1]}")
def test_layer_random_shapes(case):
    cfg, tau = case
    L, DeviceLayer = _dev()
    _check_layer(cfg, _workload(cfg), tau, L, DeviceLayer)


@pytest.mark.parametrize("case", RANDOM[::2], ids=lambda c: f"{c[0].name}-tau{c[1]}")
def test_layer_random_shapes_reuse(case):
    """The REUSE variant on every other seeded random shape."""
    cfg, tau = case
    _check_reuse(cfg, tau, expect_difference=False)


# The largest draft the boundary accepts: num_nodes * block = 16384 slots, as 256 nodes of
# 64 positions and as 16 nodes of the longest block (1024 positions: 16 key tiles of the
# branch's own block in the block phase), dense and folded.
MAXIMUM = [
    custom_config(name="max-slots-256x64-bf16", num_nodes=256, block=64, hidden=128, n_q=2,
                  n_kv=1, head_dim=64, ffn=128, prefix=16, dtype="bf16", graph="dag",
                  reveal=(1, 3), seed=95),
    custom_config(name="max-block-16x1024-f32", num_nodes=16, block=1024, hidden=128, n_q=4,
                  n_kv=2, head_dim=64, ffn=128, prefix=33, dtype="f32", graph="tree3",
                  reveal=(1, 8), seed=96),
]


@pytest.mark.parametrize("cfg", MAXIMUM, ids=lambda c: c.name)
@pytest.mark.parametrize("tau", [-1.0, 0.05])
def test_layer_maximum_sizes(cfg, tau):
    L, DeviceLayer = _dev()
    assert cfg.slots == 16384
    _check_layer(cfg, _workload(cfg), tau, L, DeviceLayer)


# The widest shapes the boundary accepts, one dimension at a time: hidden 32768 (rows of 8192
# fp32 chunks: the gate and the O finish loop over them), FFN 131072 (1639 SwiGLU slabs of
# five pairs; a down GEMM over 131072), and 256 query heads over 8 KV heads (32 query heads
# per KV head).
MAX_WIDTH = [
    custom_config(name="max-hidden-32768-f32", num_nodes=3, block=5, hidden=32768, n_q=2,
                  n_kv=1, head_dim=64, ffn=128, prefix=20, dtype="f32", graph="chain",
                  reveal=(1, 2), seed=97),
    custom_config(name="max-ffn-131072-bf16", num_nodes=2, block=9, hidden=128, n_q=2, n_kv=1,
                  head_dim=64, ffn=131072, prefix=20, dtype="bf16", graph="chain",
                  reveal=(1, 2), seed=98),
    custom_config(name="max-heads-256q8kv-bf16", num_nodes=3, block=6, hidden=256, n_q=256,
                  n_kv=8, head_dim=64, ffn=128, prefix=40, dtype="bf16", graph="tree3",
                  reveal=(1, 2), seed=99),
]


@pytest.mark.parametrize("cfg", MAX_WIDTH, ids=lambda c: c.name)
@pytest.mark.parametrize("tau", [-1.0, 0.3])
def test_layer_maximum_widths(cfg, tau):
    L, DeviceLayer = _dev()
    _check_layer(cfg, _workload(cfg), tau, L, DeviceLayer)


def test_layer_million_key_prefix():
    """A prefix of 2^20 + 37 keys (bf16; the 256-query prefix kernel over 16385 key tiles,
    the last one ragged, split across units and merged), dense and folded."""
    L, DeviceLayer = _dev()
    cfg = custom_config(name="prefix-1048613-bf16", num_nodes=3, block=5, hidden=128, n_q=4,
                        n_kv=1, head_dim=64, ffn=128, prefix=(1 << 20) + 37, dtype="bf16",
                        graph="chain", reveal=(1, 2), seed=101)
    w = _workload(cfg)
    for tau in (-1.0, 0.3):
        _check_layer(cfg, w, tau, L, DeviceLayer)
