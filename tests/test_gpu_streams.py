"""Calls on different streams (the header's concurrency contract): two layers, each with its
own workspace, fold-state and output buffers, launched interleaved on two streams of the
default priority, give the same results bit for bit as each layer run alone."""
import numpy as np
import pytest
import torch

from synth import CONFIGS, custom_config, make_workload

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from branch_folding_amd import _lib as L
    from branch_folding_amd.runner import DeviceLayer
    L.lib()
    return DeviceLayer


CASES = [
    CONFIGS[0],
    custom_config(name="streams-bf16", num_nodes=9, block=40, hidden=256, n_q=7, n_kv=1,
                  head_dim=128, ffn=384, prefix=600, dtype="bf16", graph="dag",
                  reveal=(1, 3), seed=111),
]


@pytest.mark.parametrize("tau", [0.05, -1.0])
def test_layers_on_two_streams(tau):
    DeviceLayer = _dev()
    layers = []
    for cfg in CASES:
        w = make_workload(cfg)
        layers.append(DeviceLayer(cfg, w.weights[0], w.cache, w.H, w.fold_src))
    # each layer alone, on the current stream
    ref = []
    for dl in layers:
        dl.forward(tau)
        torch.cuda.synchronize()
        ref.append((dl.out.clone(), {k: v.clone() for k, v in dl.state.items()}))
    for dl in layers:
        dl.out.fill_(7)
        for v in dl.state.values():
            v.fill_(3)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(4):                       # interleaved launches; each stream in order
        for dl, s in zip(layers, streams):
            dl.forward(tau, stream=s)
    torch.cuda.synchronize()
    for dl, (y, st) in zip(layers, ref):
        print(f"[gpu] {dl.cfg.name} tau={tau} K={int(st['packed_count'][0])}", flush=True)
        assert torch.equal(dl.out, y)
        K = int(st["packed_count"][0])
        for k in st:
            # packing writes the first K entries of packed_slot only
            got, want = (dl.state[k][:K], st[k][:K]) if k == "packed_slot" else (dl.state[k], st[k])
            assert torch.equal(got, want), k
