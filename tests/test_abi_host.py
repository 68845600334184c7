"""Host-side checks of the C ABI (CPU only; nothing here launches a kernel): the library
loads, exports every function include/specfold.h declares, sizes workspaces, and rejects
bad arguments before anything is enqueued."""
import ctypes
import math
import os
import re

import pytest

from branch_folding_amd import _lib as L
from branch_folding_amd.runner import shape_of
from synth import CONFIGS, custom_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7f0000000000          # 256-byte aligned host integer, never dereferenced


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"^\s*(?:[\w\*\s]+?)\b(specfold_\w+)\s*\(", txt, re.M))
    return names


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"specfold_gate", "specfold_resolve", "specfold_pack",
            "specfold_layer_forward"} <= names
    lib = ctypes.CDLL(L.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert L.version() >= 100


def test_workspace_sizes():
    for cfg in CONFIGS.values():
        sh = shape_of(cfg)
        n = L.specfold_layer_workspace_bytes(sh)
        S = cfg.slots
        eb = 2 if cfg.dtype == "bf16" else 4
        assert n >= S * cfg.ffn * eb + 4 * S * cfg.hidden * eb
        for which in range(4):
            off, ld = L.specfold_workspace_offset(sh, which)
            assert off % 256 == 0 and off < n and ld >= cfg.hidden
    assert L.specfold_layer_workspace_bytes(shape_of(CONFIGS[1], prefix_len=0)) > 0


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 96, L.SPECFOLD_ERR_UNSUPPORTED),
    ("hidden", 200, L.SPECFOLD_ERR_UNSUPPORTED),
    ("ffn", 100, L.SPECFOLD_ERR_UNSUPPORTED),
    ("n_kv_heads", 3, L.SPECFOLD_ERR_INVALID_ARGUMENT),
    ("num_nodes", 0, L.SPECFOLD_ERR_INVALID_ARGUMENT),
    ("block", 2000, L.SPECFOLD_ERR_UNSUPPORTED),
    ("num_nodes", 600, L.SPECFOLD_ERR_UNSUPPORTED),      # 600 * 32 slots > 16384
    ("dtype", 7, L.SPECFOLD_ERR_INVALID_ARGUMENT),
    ("prefix_len", -1, L.SPECFOLD_ERR_INVALID_ARGUMENT),
    ("rms_eps", float("nan"), L.SPECFOLD_ERR_INVALID_ARGUMENT),
])
def test_bad_shapes_rejected(field, value, status):
    sh = shape_of(CONFIGS[1])
    setattr(sh, field, value)
    assert L.lib().specfold_layer_workspace_bytes(ctypes.byref(sh)) == 0
    assert L.last_error()
    rc = L.lib().specfold_layer_forward(ctypes.byref(sh), None, None, FAKE, FAKE + (1 << 30), FAKE,
                                        0.05, None, 0, FAKE, 1 << 40, None)
    assert rc == status, L.last_error()


def _weights(ptr=FAKE):
    return {k: ptr for k in ("rms1", "w_qkv", "w_o", "rms2", "w_gate_up", "w_down")}


def _fwd(sh, **kw):
    args = dict(weights=_weights(), prefix=(FAKE, FAKE, 1024, 128), hidden_in=FAKE,
                hidden_out=FAKE + (1 << 32), fold_src=FAKE, tau=0.05, state=None, flags=0,
                workspace=FAKE, workspace_bytes=1 << 40)
    args.update(kw)
    with pytest.raises(L.SpecFoldError) as e:
        L.specfold_layer_forward(sh, args["weights"], args["prefix"], args["hidden_in"],
                                 args["hidden_out"], args["fold_src"], args["tau"],
                                 args["state"], args["flags"], args["workspace"],
                                 args["workspace_bytes"], stream=0)
    return e.value.status, str(e.value)


def test_forward_argument_errors():
    sh = shape_of(CONFIGS[1])
    need = L.specfold_layer_workspace_bytes(sh)
    w = _weights()
    w["w_o"] = None
    assert _fwd(sh, weights=w)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    w = _weights()
    w["w_down"] = FAKE + 8                                       # misaligned
    assert _fwd(sh, weights=w)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    assert _fwd(sh, hidden_out=FAKE)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT          # aliasing
    assert _fwd(sh, hidden_in=None)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    assert _fwd(sh, prefix=None)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    assert _fwd(sh, prefix=(FAKE, FAKE, 1001, 128))[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    # token strides the prefix kernels cannot address (bf16: 2^25 elements = 64 MB)
    assert _fwd(sh, prefix=(FAKE, FAKE, 1 << 25, 128))[0] == L.SPECFOLD_ERR_UNSUPPORTED
    # just below it the view passes, and the call fails on the next check (no fold_src)
    st, msg = _fwd(sh, prefix=(FAKE, FAKE, (1 << 25) - 8, 128), fold_src=None)
    assert st == L.SPECFOLD_ERR_INVALID_ARGUMENT and "fold_src" in msg
    assert _fwd(sh, fold_src=None)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    assert _fwd(sh, flags=4)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    assert _fwd(sh, flags=L.SPECFOLD_FLAG_FOLD_STATE_IN,
                state={"recompute": FAKE})[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    assert _fwd(sh, workspace_bytes=need - 1)[0] == L.SPECFOLD_ERR_WORKSPACE
    assert _fwd(sh, workspace=None)[0] == L.SPECFOLD_ERR_WORKSPACE
    assert _fwd(sh, workspace=FAKE + 16)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT


def test_fold_step_argument_errors():
    sh = shape_of(CONFIGS[0])
    with pytest.raises(L.SpecFoldError):
        L.specfold_gate(sh, FAKE, FAKE, 0.05, None, None, stream=0)
    with pytest.raises(L.SpecFoldError):
        L.specfold_gate(sh, FAKE + 4, FAKE, 0.05, None, FAKE, stream=0)
    with pytest.raises(L.SpecFoldError):
        L.specfold_resolve(sh, FAKE, None, FAKE, stream=0)
    with pytest.raises(L.SpecFoldError):
        L.specfold_pack(sh, FAKE, FAKE, FAKE, None, FAKE, stream=0)
    bad = shape_of(custom_config(block=0))
    with pytest.raises(L.SpecFoldError):
        L.specfold_pack(bad, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)


def _stack(sh, n=3, **kw):
    args = dict(weights=[_weights() for _ in range(n)],
                prefix=[(FAKE, FAKE, 1024, 128) for _ in range(n)], hidden_in=FAKE,
                hidden_out=FAKE + (1 << 32), fold_src=FAKE, tau=0.05, states=None, flags=0,
                workspace=FAKE + (1 << 34), workspace_bytes=1 << 40, num_layers=None)
    args.update(kw)
    with pytest.raises(L.SpecFoldError) as e:
        L.specfold_stack_forward(sh, args["weights"], args["prefix"], args["hidden_in"],
                                 args["hidden_out"], args["fold_src"], args["tau"],
                                 args["states"], args["flags"], args["workspace"],
                                 args["workspace_bytes"], stream=0,
                                 num_layers=args["num_layers"])
    return e.value.status, str(e.value)


def test_stack_workspace_holds_a_layer_and_a_hidden_buffer():
    for cfg in CONFIGS.values():
        sh = shape_of(cfg)
        eb = 2 if cfg.dtype == "bf16" else 4
        assert (L.specfold_stack_workspace_bytes(sh)
                == L.specfold_layer_workspace_bytes(sh) + cfg.slots * cfg.hidden * eb)


def test_stack_argument_errors():
    sh = shape_of(CONFIGS[3])
    need = L.specfold_stack_workspace_bytes(sh)
    assert _stack(sh, weights=[])[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT        # 0 layers
    w = [_weights() for _ in range(3)]
    w[2]["w_qkv"] = None
    st, msg = _stack(sh, weights=w)
    assert st == L.SPECFOLD_ERR_INVALID_ARGUMENT and "layer 2" in msg
    p = [(FAKE, FAKE, 1024, 128)] * 3
    p[1] = (FAKE, FAKE + 2, 1024, 128)                                          # misaligned
    st, msg = _stack(sh, prefix=p)
    assert st == L.SPECFOLD_ERR_INVALID_ARGUMENT and "layer 1" in msg
    assert _stack(sh, prefix=None)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    assert _stack(sh, hidden_out=FAKE)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    assert _stack(sh, fold_src=None)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    assert _stack(sh, flags=L.SPECFOLD_FLAG_FOLD_STATE_IN)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    full = {k: FAKE for k in ("recompute", "src_node", "packed_slot", "slot_row", "packed_count")}
    st, msg = _stack(sh, flags=L.SPECFOLD_FLAG_FOLD_STATE_IN,
                     states=[full, full, {"recompute": FAKE}])
    assert st == L.SPECFOLD_ERR_INVALID_ARGUMENT and "layer 2" in msg
    assert _stack(sh, workspace_bytes=need - 1)[0] == L.SPECFOLD_ERR_WORKSPACE
    # hidden buffers inside the workspace
    assert _stack(sh, hidden_in=FAKE + (1 << 34) + 4096)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    assert _stack(sh, hidden_out=FAKE + (1 << 34) + need - 256)[0] == L.SPECFOLD_ERR_INVALID_ARGUMENT
    # no prefix views needed without a prefix
    sh0 = shape_of(CONFIGS[3], prefix_len=0)
    assert _stack(sh0, prefix=None, workspace_bytes=0)[0] == L.SPECFOLD_ERR_WORKSPACE


def test_lm_head_workspace_and_argument_errors():
    sh = shape_of(CONFIGS[1])
    V = 152064
    ws = L.specfold_lm_head_workspace_bytes(sh, V)
    S, d = CONFIGS[1].slots, CONFIGS[1].hidden
    P = -(-V // 128) * 2
    assert ws >= S * (d + 64) * 2 + 2 * S * P * 4
    assert L.lib().specfold_lm_head_workspace_bytes(ctypes.byref(sh), 0) == 0
    args = [FAKE] * 9
    # every case below fails in the host-side checks, before anything is enqueued
    def call(vocab=V, ptrs=None, wsb=ws, shape=sh):
        p = list(args if ptrs is None else ptrs)
        assert len(p) == 9
        return L.lib().specfold_lm_head_argmax(ctypes.byref(shape), vocab, *p, FAKE, wsb, None)
    assert call(vocab=0) == L.SPECFOLD_ERR_INVALID_ARGUMENT
    for i in (0, 1, 2, 3, 4, 5, 6, 8):        # every pointer but row_logit is required
        bad = list(args)
        bad[i] = None
        assert call(ptrs=bad) == L.SPECFOLD_ERR_INVALID_ARGUMENT, i
    bad = list(args)
    bad[1] = FAKE + 8                         # misaligned weight
    assert call(ptrs=bad) == L.SPECFOLD_ERR_INVALID_ARGUMENT
    assert call(wsb=ws - 1) == L.SPECFOLD_ERR_WORKSPACE
    odd = shape_of(CONFIGS[1])
    odd.hidden = 3600
    assert call(shape=odd) == L.SPECFOLD_ERR_UNSUPPORTED
