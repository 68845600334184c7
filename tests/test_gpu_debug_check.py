"""The draft-graph check of SPECFOLD_DEBUG mode on the GPU: a fold_src entry that breaks the
topological numbering (the root's not -1, or node n's outside [0, n)) makes the call fail
with SPECFOLD_ERR_INVALID_ARGUMENT naming the first such node, before any of the call's
kernels run; a well-formed graph gives the same output, bit for bit, as without the check."""
import numpy as np
import pytest
import torch

from synth import CONFIGS, make_workload


@pytest.mark.gpu
def test_debug_check_of_the_draft_graph(monkeypatch):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from branch_folding_amd import _lib as L
    from branch_folding_amd.runner import DeviceLayer, DeviceStack, shape_of
    cfg = CONFIGS[0]
    w = make_workload(cfg, layers=2)
    N = cfg.num_nodes
    print(f"[gpu] debug check {cfg.name}", flush=True)
    monkeypatch.delenv("SPECFOLD_DEBUG", raising=False)
    dl = DeviceLayer(cfg, w.weights[0], w.cache, w.H, w.fold_src)
    ref = dl.forward(0.05).clone()
    torch.cuda.synchronize()

    monkeypatch.setenv("SPECFOLD_DEBUG", "1")
    out = dl.forward(0.05, out=torch.empty_like(ref))
    torch.cuda.synchronize()
    assert torch.equal(out, ref)

    good = np.asarray(w.fold_src, dtype=np.int32)
    sh = shape_of(cfg)
    rec = torch.empty(cfg.slots, dtype=torch.uint8, device="cuda")
    src = torch.empty(cfg.slots, dtype=torch.int32, device="cuda")
    for node, val in ((0, 0), (N - 1, N - 1), (N // 2, -3), (1, N + 5)):
        bad = good.copy()
        bad[node] = val
        dl.fold_src.copy_(torch.from_numpy(bad))
        sentinel = torch.full_like(ref, 7.0)
        with pytest.raises(L.SpecFoldError) as e:
            dl.forward(0.05, out=sentinel)
        assert e.value.status == L.SPECFOLD_ERR_INVALID_ARGUMENT
        assert f"fold_src[{node}] = {val}" in str(e.value)
        torch.cuda.synchronize()
        assert bool((sentinel == 7.0).all()), "a layer kernel ran despite the failed check"
        with pytest.raises(L.SpecFoldError):
            L.specfold_gate(sh, dl.H, dl.fold_src, 0.05, None, rec)
        with pytest.raises(L.SpecFoldError):
            L.specfold_resolve(sh, rec, dl.fold_src, src)
    dl.fold_src.copy_(torch.from_numpy(good))

    # a stack checks the graph once, before its first layer
    ds = DeviceStack(cfg, [], w.H, good)
    for l in range(2):
        ds.add_layer(w.weights[l], w.caches[l])
    y_ok = ds.forward(0.05).clone()
    ds.fold_src.copy_(torch.from_numpy(np.where(np.arange(N) == 2, 2, good).astype(np.int32)))
    with pytest.raises(L.SpecFoldError) as e:
        ds.forward(0.05)
    assert "fold_src[2] = 2" in str(e.value)
    monkeypatch.delenv("SPECFOLD_DEBUG")
    ds.fold_src.copy_(torch.from_numpy(good))
    torch.cuda.synchronize()
    assert torch.equal(ds.forward(0.05), y_ok)
