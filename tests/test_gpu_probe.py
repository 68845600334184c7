"""Timing probes of specfold_layer_forward_probed: a probe on any step leaves the layer's
outputs bit for bit as they are without it, records its event pair for every step the call
runs (the FFN gate/up step through hipExtLaunchKernel when it is one kernel), and records
nothing for a step the call skips."""
import ctypes

import numpy as np
import pytest
import torch

from synth import CONFIGS, custom_config, make_workload

pytestmark = pytest.mark.gpu


class _Events:
    """hipEvent_t create / elapsed through the HIP runtime that torch has loaded."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so.7")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def ms(self, a, b):
        assert self.h.hipEventSynchronize(b) == 0
        v = ctypes.c_float()
        if self.h.hipEventElapsedTime(ctypes.byref(v), a, b) != 0:
            self.h.hipGetLastError()
            return None
        return v.value

    def destroy(self, *evs):
        for e in evs:
            self.h.hipEventDestroy(e)


CASES = [
    CONFIGS[0],                                                    # fp32, slab SwiGLU
    custom_config(name="probe-bf16", num_nodes=6, block=32, hidden=256, n_q=4, n_kv=2,
                  head_dim=128, ffn=512, prefix=200, dtype="bf16", graph="tree3",
                  reveal=(1, 2), seed=71),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_probe_every_step(cfg):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from branch_folding_amd import _lib as L
    from branch_folding_amd.runner import DeviceLayer
    L.lib()
    print(f"probe case {cfg.name}", flush=True)
    w = make_workload(cfg, layers=1)
    dl = DeviceLayer(cfg, w.weights[0], w.cache, w.H, w.fold_src)
    stream = torch.cuda.current_stream().cuda_stream
    ref = dl.forward(cfg.tau, stream=stream).clone()
    torch.cuda.synchronize()
    ev = _Events()
    times = {}
    for idx, name in enumerate(L.STEPS):
        a, b = ev.create(), ev.create()
        out = dl.forward(cfg.tau, stream=stream, probe=L.Probe(idx, a, b))
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"step {name}: a probe changed the output"
        times[name] = ev.ms(a, b)
        ev.destroy(a, b)
    # steps every call of these shapes runs (the others are fused into a neighbour or skipped)
    for name in ("gate", "resolve_pack", "qkv", "attn_block", "o_proj", "o_finish",
                 "ffn_gate_up", "ffn_down", "combine"):
        t = times[name]
        assert t is not None and np.isfinite(t) and 0.0 <= t < 50.0, (name, t)
    assert times["rmsnorm1"] is None          # fused into the gate: nothing recorded
