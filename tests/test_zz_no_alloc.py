"""The allocation-free layer entry point (specfold_layer_forward_static: the workspace is
a static device array inside the library) against specfold_layer_forward with a caller
workspace, through the C ABI.  Both run the same launches on the same inputs, so outputs
and fold states must be bit-identical; two calls in a row, the second on a smaller layer,
so the second runs on the array the first left behind."""
import numpy as np
import pytest
import torch

from synth import CONFIGS, budget_config, make_workload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _run_both(cfg, tau, L, DeviceLayer, reuse=False):
    w = make_workload(cfg)
    dl = DeviceLayer(cfg, w.weights[0], w.cache, w.H, w.fold_src)
    flags = L.SPECFOLD_FLAG_REUSE_ATTENTION if reuse else 0
    _say(f"[gpu] static workspace {cfg.name} tau={tau} reuse={reuse} "
         f"(workspace {dl.ws_bytes >> 20} MiB of {L.SPECFOLD_STATIC_WORKSPACE_BYTES >> 20})")
    dl.forward(tau, reuse=reuse)
    torch.cuda.synchronize()
    y_ref = dl.out.clone()
    st_ref = dl.fold_state()
    out = torch.full_like(dl.out, 3.0)
    st = {k: torch.full_like(v, 7) for k, v in dl.state.items()}
    L.specfold_layer_forward_static(dl.shape, dl.w, dl.prefix, dl.H, out, dl.fold_src, tau,
                                    st, flags)
    torch.cuda.synchronize()
    assert torch.equal(out, y_ref)
    K = int(st["packed_count"][0].item())
    assert K == st_ref["K"]
    N, B = cfg.num_nodes, cfg.block
    np.testing.assert_array_equal(st["recompute"].cpu().numpy().reshape(N, B) != 0,
                                  st_ref["recompute"])
    np.testing.assert_array_equal(st["src_node"].cpu().numpy().reshape(N, B), st_ref["src"])
    np.testing.assert_array_equal(st["packed_slot"].cpu().numpy()[:K], st_ref["packed_slot"])
    np.testing.assert_array_equal(st["slot_row"].cpu().numpy().reshape(N, B),
                                  st_ref["slot_row"])
    np.testing.assert_array_equal(st["ratio"].cpu().numpy().reshape(N, B), st_ref["ratio"])
    _say(f"[gpu]   K={K}: output and fold state bit-identical")


def test_static_workspace_layer_equals_workspace_layer():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from branch_folding_amd import _lib as L
    from branch_folding_amd.runner import DeviceLayer
    L.lib()
    # the 7B-shaped benchmark layer, then a smaller one (1 + 3 branches) and the tiny fp32
    # layer, each on what the previous call left in the array
    _run_both(CONFIGS[1], CONFIGS[1].tau, L, DeviceLayer)
    _run_both(budget_config(4), 0.05, L, DeviceLayer)
    _run_both(CONFIGS[0], CONFIGS[0].tau, L, DeviceLayer, reuse=True)


def test_static_workspace_rejects_oversized_shapes():
    """A shape whose workspace exceeds the static array is refused before any launch."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from branch_folding_amd import _lib as L
    from branch_folding_amd.runner import shape_of
    L.lib()
    cfg = CONFIGS[4]
    sh = shape_of(cfg)
    assert L.specfold_layer_workspace_bytes(sh) > L.SPECFOLD_STATIC_WORKSPACE_BYTES
    fake = torch.empty(16, dtype=torch.uint8, device="cuda")
    w = {k: fake for k in ("rms1", "w_qkv", "w_o", "rms2", "w_gate_up", "w_down")}
    out = torch.empty(cfg.slots * cfg.hidden, dtype=torch.bfloat16, device="cuda")
    hin = torch.empty_like(out)
    with pytest.raises(L.SpecFoldError) as e:
        L.specfold_layer_forward_static(sh, w, (fake, fake, 2 * cfg.n_kv * cfg.head_dim,
                                                cfg.head_dim), hin, out, fake, 0.02)
    assert e.value.status == L.SPECFOLD_ERR_WORKSPACE
    torch.cuda.synchronize()
