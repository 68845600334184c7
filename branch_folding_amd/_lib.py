"""ctypes binding of libspecfold.so: the C ABI of include/specfold.h, same names, argument
marshalling only.  Every step of the layer runs in the HIP library; torch tensors are used
only as device buffers and streams.  Loading fails loudly when the library is missing."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspecfold.so")

SPECFOLD_OK = 0
SPECFOLD_ERR_INVALID_ARGUMENT = 1
SPECFOLD_ERR_UNSUPPORTED = 2
SPECFOLD_ERR_WORKSPACE = 3
SPECFOLD_ERR_HIP = 4
SPECFOLD_F32 = 0
SPECFOLD_BF16 = 1
SPECFOLD_FLAG_FOLD_STATE_IN = 1
SPECFOLD_FLAG_REUSE_ATTENTION = 2
SPECFOLD_T_QKV, SPECFOLD_T_ATTN, SPECFOLD_T_H, SPECFOLD_T_FFN = 0, 1, 2, 3

_STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "WORKSPACE", 4: "HIP"}


class SpecFoldError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"specfold {_STATUS.get(status, status)}: {message}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("num_nodes", ctypes.c_int32), ("block", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("prefix_len", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("rope_theta", ctypes.c_float)]


class KVView(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("stride_tok", ctypes.c_int64), ("stride_head", ctypes.c_int64)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("rms1", ctypes.c_void_p), ("w_qkv", ctypes.c_void_p), ("w_o", ctypes.c_void_p),
                ("rms2", ctypes.c_void_p), ("w_gate_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("b_qkv", ctypes.c_void_p)]


class Probe(ctypes.Structure):
    _fields_ = [("step", ctypes.c_int32), ("start", ctypes.c_void_p), ("stop", ctypes.c_void_p)]


STEPS = ["gate", "resolve_pack", "rmsnorm1", "qkv", "attn_prefix", "attn_block", "o_proj",
         "o_finish", "ffn_gate_up", "ffn_down", "combine"]


class FoldState(ctypes.Structure):
    _fields_ = [("ratio", ctypes.c_void_p), ("recompute", ctypes.c_void_p),
                ("src_node", ctypes.c_void_p), ("packed_slot", ctypes.c_void_p),
                ("slot_row", ctypes.c_void_p), ("packed_count", ctypes.c_void_p)]


_lib = None
_P = ctypes.c_void_p
_SIGS = {
    "specfold_gate": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, ctypes.c_float, _P, _P, _P]),
    "specfold_resolve": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P]),
    "specfold_pack": (ctypes.c_int, [ctypes.POINTER(Shape), _P, _P, _P, _P, _P, _P]),
    "specfold_layer_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Shape)]),
    "specfold_layer_forward": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.POINTER(LayerWeights),
                                              ctypes.POINTER(KVView), _P, _P, _P, ctypes.c_float,
                                              ctypes.POINTER(FoldState), ctypes.c_uint32, _P,
                                              ctypes.c_size_t, _P]),
    "specfold_layer_forward_probed": (ctypes.c_int, [ctypes.POINTER(Shape),
                                                     ctypes.POINTER(LayerWeights),
                                                     ctypes.POINTER(KVView), _P, _P, _P,
                                                     ctypes.c_float, ctypes.POINTER(FoldState),
                                                     ctypes.c_uint32, _P, ctypes.c_size_t, _P,
                                                     ctypes.POINTER(Probe)]),
    "specfold_layer_forward_static": (ctypes.c_int, [ctypes.POINTER(Shape),
                                                     ctypes.POINTER(LayerWeights),
                                                     ctypes.POINTER(KVView), _P, _P, _P,
                                                     ctypes.c_float, ctypes.POINTER(FoldState),
                                                     ctypes.c_uint32, _P]),
    "specfold_workspace_offset": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32,
                                                     ctypes.POINTER(ctypes.c_int64)]),
    "specfold_stack_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Shape)]),
    "specfold_stack_forward": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_int32,
                                              ctypes.POINTER(LayerWeights),
                                              ctypes.POINTER(KVView), _P, _P, _P,
                                              ctypes.c_float, ctypes.POINTER(FoldState),
                                              ctypes.c_uint32, _P, ctypes.c_size_t, _P]),
    "specfold_lm_head_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Shape), ctypes.c_int32]),
    "specfold_lm_head_argmax": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_int32, _P, _P, _P,
                                               _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "specfold_last_error": (ctypes.c_char_p, []),
    "specfold_version": (ctypes.c_int32, []),
}


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch first: the library then binds to the HIP runtime torch has loaded (same
        # soname), so both share one runtime and one set of streams.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m branch_folding_amd.build` (there is no fallback)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def last_error() -> str:
    return lib().specfold_last_error().decode()


def version() -> int:
    return int(lib().specfold_version())


def _check(status: int) -> None:
    if status != SPECFOLD_OK:
        raise SpecFoldError(status, last_error())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_shape(num_nodes, block, hidden, n_q, n_kv, head_dim, ffn, prefix, dtype,
               rms_eps=1e-6, rope_theta=0.0) -> Shape:
    dt = {"f32": SPECFOLD_F32, "bf16": SPECFOLD_BF16}.get(dtype, dtype)
    return Shape(num_nodes, block, hidden, n_q, n_kv, head_dim, ffn, prefix, rms_eps, dt,
                 rope_theta)


def specfold_gate(shape: Shape, hidden, fold_src, tau: float, ratio, recompute, stream=None):
    _check(lib().specfold_gate(ctypes.byref(shape), _ptr(hidden), _ptr(fold_src), float(tau),
                               _ptr(ratio), _ptr(recompute), _stream(stream)))


def specfold_resolve(shape: Shape, recompute, fold_src, src_node, stream=None):
    _check(lib().specfold_resolve(ctypes.byref(shape), _ptr(recompute), _ptr(fold_src),
                                  _ptr(src_node), _stream(stream)))


def specfold_pack(shape: Shape, recompute, src_node, packed_slot, slot_row, packed_count,
                  stream=None):
    _check(lib().specfold_pack(ctypes.byref(shape), _ptr(recompute), _ptr(src_node),
                               _ptr(packed_slot), _ptr(slot_row), _ptr(packed_count),
                               _stream(stream)))


def specfold_lm_head_workspace_bytes(shape: Shape, vocab: int) -> int:
    n = int(lib().specfold_lm_head_workspace_bytes(ctypes.byref(shape), int(vocab)))
    if n == 0:
        raise SpecFoldError(SPECFOLD_ERR_INVALID_ARGUMENT, last_error())
    return n


def specfold_lm_head_argmax(shape: Shape, vocab: int, rms_final, w_lm, hidden, packed_slot,
                            slot_row, packed_count, row_token, row_logit, token, workspace,
                            workspace_bytes: int, stream=None):
    _check(lib().specfold_lm_head_argmax(ctypes.byref(shape), int(vocab), _ptr(rms_final),
                                         _ptr(w_lm), _ptr(hidden), _ptr(packed_slot),
                                         _ptr(slot_row), _ptr(packed_count), _ptr(row_token),
                                         _ptr(row_logit), _ptr(token), _ptr(workspace),
                                         int(workspace_bytes), _stream(stream)))


def specfold_layer_workspace_bytes(shape: Shape) -> int:
    n = int(lib().specfold_layer_workspace_bytes(ctypes.byref(shape)))
    if n == 0:
        raise SpecFoldError(SPECFOLD_ERR_INVALID_ARGUMENT, last_error())
    return n


def specfold_workspace_offset(shape: Shape, which: int):
    """(byte offset, row stride in elements) of a workspace intermediate."""
    ld = ctypes.c_int64(0)
    off = int(lib().specfold_workspace_offset(ctypes.byref(shape), int(which), ctypes.byref(ld)))
    if off == ctypes.c_size_t(-1).value:
        raise SpecFoldError(SPECFOLD_ERR_INVALID_ARGUMENT, last_error())
    return off, int(ld.value)


_WEIGHT_KEYS = ("rms1", "w_qkv", "w_o", "rms2", "w_gate_up", "w_down")
_STATE_KEYS = ("ratio", "recompute", "src_node", "packed_slot", "slot_row", "packed_count")


def _weights(weights: dict) -> LayerWeights:
    w = LayerWeights(*[_ptr(weights[k]) for k in _WEIGHT_KEYS])
    if weights.get("b_qkv") is not None:
        w.b_qkv = _ptr(weights["b_qkv"])
    return w


def _kv(prefix) -> KVView:
    if prefix is None:
        return KVView(None, None, 0, 0)
    return KVView(_ptr(prefix[0]), _ptr(prefix[1]), int(prefix[2]), int(prefix[3]))


def _state(state: dict) -> FoldState:
    return FoldState(*[_ptr(state.get(k)) for k in _STATE_KEYS])


def specfold_layer_forward(shape: Shape, weights: dict, prefix, hidden_in, hidden_out,
                           fold_src, tau: float, state: Optional[dict] = None, flags: int = 0,
                           workspace=None, workspace_bytes: Optional[int] = None, stream=None,
                           probe: Optional[Probe] = None):
    """weights: dict of device tensors rms1, w_qkv, w_o, rms2, w_gate_up, w_down.
    prefix: (k_ptr_or_tensor, v_ptr_or_tensor, stride_tok, stride_head) or None.
    state: dict with any of ratio, recompute, src_node, packed_slot, slot_row, packed_count."""
    lw = _weights(weights)
    kv = _kv(prefix)
    st = None if state is None else _state(state)
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (ctypes.byref(shape), ctypes.byref(lw), ctypes.byref(kv), _ptr(hidden_in),
            _ptr(hidden_out), _ptr(fold_src), float(tau),
            ctypes.byref(st) if st is not None else None, int(flags), _ptr(workspace),
            int(workspace_bytes), _stream(stream))
    if probe is None:
        _check(lib().specfold_layer_forward(*args))
    else:
        _check(lib().specfold_layer_forward_probed(*args, ctypes.byref(probe)))


SPECFOLD_STATIC_WORKSPACE_BYTES = 128 << 20


def specfold_layer_forward_static(shape: Shape, weights: dict, prefix, hidden_in, hidden_out,
                                  fold_src, tau: float, state: Optional[dict] = None,
                                  flags: int = 0, stream=None):
    """specfold_layer_forward with the library's static device workspace (no workspace
    argument; the call allocates nothing)."""
    lw = _weights(weights)
    kv = _kv(prefix)
    st = None if state is None else _state(state)
    _check(lib().specfold_layer_forward_static(
        ctypes.byref(shape), ctypes.byref(lw), ctypes.byref(kv), _ptr(hidden_in),
        _ptr(hidden_out), _ptr(fold_src), float(tau),
        ctypes.byref(st) if st is not None else None, int(flags), _stream(stream)))


def specfold_stack_workspace_bytes(shape: Shape) -> int:
    n = int(lib().specfold_stack_workspace_bytes(ctypes.byref(shape)))
    if n == 0:
        raise SpecFoldError(SPECFOLD_ERR_INVALID_ARGUMENT, last_error())
    return n


def specfold_stack_forward(shape: Shape, weights: list, prefix, hidden_in, hidden_out,
                           fold_src, tau: float, states: Optional[list] = None,
                           flags: int = 0, workspace=None,
                           workspace_bytes: Optional[int] = None, stream=None,
                           num_layers: Optional[int] = None):
    """weights: list of per-layer weight dicts (as specfold_layer_forward's); prefix: list
    of per-layer views or None; states: list of per-layer state dicts or None."""
    nl = len(weights) if num_layers is None else int(num_layers)
    wa = (LayerWeights * max(len(weights), 1))(*[_weights(w) for w in weights])
    pa = None
    if prefix is not None:
        pa = (KVView * max(len(prefix), 1))(*[_kv(p) for p in prefix])
    sa = None
    if states is not None:
        sa = (FoldState * max(len(states), 1))(*[_state(st) for st in states])
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().specfold_stack_forward(
        ctypes.byref(shape), nl, wa, pa, _ptr(hidden_in), _ptr(hidden_out), _ptr(fold_src),
        float(tau), sa, int(flags), _ptr(workspace), int(workspace_bytes), _stream(stream)))
