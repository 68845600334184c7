"""Device-side marshalling of a synthetic workload for the C ABI (no layer arithmetic).

Uploads weights, the interleaved prefix cache, hidden states and the draft graph to the
GPU once, allocates the output, fold-state and workspace buffers, and calls
specfold_layer_forward through the binding.  Used by the GPU tests, the smoke check and
the benchmark."""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import _lib as L


def torch_dtype(cfg) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def to_device(x: np.ndarray, dtype: torch.dtype, device) -> torch.Tensor:
    """Exact upload: bf16 configs carry bf16-representable fp32 values."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device=device, dtype=dtype)


def _as_device(x, dtype: torch.dtype, device) -> torch.Tensor:
    """A host array uploaded exactly, or a tensor already drawn on the device (converted
    to the layer's dtype)."""
    if isinstance(x, torch.Tensor):
        return x.to(device=device, dtype=dtype).contiguous()
    return to_device(x, dtype, device)


def shape_of(cfg, prefix_len: Optional[int] = None) -> L.Shape:
    return L.make_shape(cfg.num_nodes, cfg.block, cfg.hidden, cfg.n_q, cfg.n_kv, cfg.head_dim,
                        cfg.ffn, cfg.prefix if prefix_len is None else prefix_len, cfg.dtype,
                        cfg.rms_eps, cfg.rope_theta)


class DeviceLayer:
    """One verify layer's inputs and buffers resident in HBM."""

    def __init__(self, cfg, weights: Dict[str, np.ndarray], cache: np.ndarray, H: np.ndarray,
                 fold_src: np.ndarray, device="cuda:0"):
        self.cfg = cfg
        self.device = torch.device(device)
        dt = torch_dtype(cfg)
        self.dt = dt
        self.shape = shape_of(cfg)
        self.w = {k: to_device(v, dt, self.device) for k, v in weights.items()}
        self.cache = to_device(cache, dt, self.device)           # [P+pad, 2, n_kv, dh]
        S, d = cfg.slots, cfg.hidden
        self.H = to_device(H.reshape(S, d), dt, self.device)
        self.out = torch.empty((S, d), dtype=dt, device=self.device)
        self.fold_src = torch.from_numpy(np.asarray(fold_src, dtype=np.int32)).to(self.device)
        self.state = {
            "ratio": torch.empty(S, dtype=torch.float32, device=self.device),
            "recompute": torch.empty(S, dtype=torch.uint8, device=self.device),
            "src_node": torch.empty(S, dtype=torch.int32, device=self.device),
            "packed_slot": torch.empty(S, dtype=torch.int32, device=self.device),
            "slot_row": torch.empty(S, dtype=torch.int32, device=self.device),
            "packed_count": torch.zeros(1, dtype=torch.int32, device=self.device),
        }
        self.ws_bytes = L.specfold_layer_workspace_bytes(self.shape)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        n_kv, dh = cfg.n_kv, cfg.head_dim
        self.prefix = (self.cache[0, 0].data_ptr(), self.cache[0, 1].data_ptr(),
                       2 * n_kv * dh, dh)

    def set_hidden(self, H) -> None:
        if isinstance(H, torch.Tensor):
            self.H.copy_(H.reshape(self.H.shape))
        else:
            self.H.copy_(to_device(H.reshape(self.H.shape), self.dt, self.device))

    def forward(self, tau: float, stream=None, state_in: Optional[Dict[str, np.ndarray]] = None,
                out: Optional[torch.Tensor] = None, probe=None, reuse: bool = False
                ) -> torch.Tensor:
        flags = L.SPECFOLD_FLAG_REUSE_ATTENTION if reuse else 0
        if state_in is not None:
            for k in ("recompute", "src_node", "packed_slot", "slot_row", "packed_count"):
                v = np.asarray(state_in[k]).reshape(-1)
                self.state[k].copy_(torch.from_numpy(v.astype(
                    np.uint8 if k == "recompute" else np.int32)).to(self.device))
            flags |= L.SPECFOLD_FLAG_FOLD_STATE_IN
        o = self.out if out is None else out
        L.specfold_layer_forward(self.shape, self.w, self.prefix, self.H, o, self.fold_src, tau,
                                 self.state, flags, self.ws, self.ws_bytes, stream, probe)
        return o

    def fold_state(self) -> Dict[str, np.ndarray]:
        N, B = self.cfg.num_nodes, self.cfg.block
        st = {k: v.cpu().numpy() for k, v in self.state.items()}
        K = int(st["packed_count"][0])
        return dict(ratio=st["ratio"].reshape(N, B), recompute=st["recompute"].reshape(N, B) != 0,
                    src=st["src_node"].reshape(N, B), packed_slot=st["packed_slot"][:K],
                    slot_row=st["slot_row"].reshape(N, B), K=K)

    def intermediate(self, which: int) -> torch.Tensor:
        """View of a workspace tensor after the stream has synchronised."""
        cfg = self.cfg
        off, ld = L.specfold_workspace_offset(self.shape, which)
        S = cfg.slots
        cols = {L.SPECFOLD_T_QKV: cfg.qkv_dim, L.SPECFOLD_T_ATTN: cfg.n_q * cfg.head_dim,
                L.SPECFOLD_T_H: cfg.hidden, L.SPECFOLD_T_FFN: cfg.hidden}[which]
        es = torch.tensor([], dtype=self.dt).element_size()
        return self.ws[off: off + S * ld * es].view(self.dt).view(S, ld)[:, :cols]

    def output_numpy(self) -> np.ndarray:
        cfg = self.cfg
        return self.out.float().cpu().numpy().reshape(cfg.num_nodes, cfg.block, cfg.hidden)


class DeviceStack:
    """A stack of verify layers resident in HBM: per-layer weights and prefix caches, the
    input hidden states, per-layer fold-state buffers and the stack workspace."""

    def __init__(self, cfg, layers, H: np.ndarray, fold_src: np.ndarray, device="cuda:0"):
        """layers: iterable of (weights dict, interleaved prefix cache) per layer; each is
        uploaded as it is produced, so host memory holds one layer at a time.  More layers
        can be appended with add_layer() before the first call."""
        self.cfg = cfg
        self.device = torch.device(device)
        dt = torch_dtype(cfg)
        self.dt = dt
        self.shape = shape_of(cfg)
        self.w, self.caches, self.prefix, self.states = [], [], [], []
        S, d = cfg.slots, cfg.hidden
        self.H = to_device(H.reshape(S, d), dt, self.device)
        self.out = torch.empty((S, d), dtype=dt, device=self.device)
        self.fold_src = torch.from_numpy(np.asarray(fold_src, dtype=np.int32)).to(self.device)
        for weights, cache in layers:
            self.add_layer(weights, cache)
        self.ws_bytes = L.specfold_stack_workspace_bytes(self.shape)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)

    @property
    def num_layers(self) -> int:
        return len(self.w)

    def add_layer(self, weights: Dict[str, np.ndarray], cache: np.ndarray) -> None:
        """Upload one more layer's weights and prefix cache (host arrays, or tensors drawn
        on the device), with its fold-state buffers."""
        cfg, dt, S = self.cfg, self.dt, self.cfg.slots
        n_kv, dh = cfg.n_kv, cfg.head_dim
        self.w.append({k: _as_device(v, dt, self.device) for k, v in weights.items()})
        c = _as_device(cache, dt, self.device)
        self.caches.append(c)
        self.prefix.append((c[0, 0].data_ptr(), c[0, 1].data_ptr(), 2 * n_kv * dh, dh))
        self.states.append({
            "ratio": torch.empty(S, dtype=torch.float32, device=self.device),
            "recompute": torch.empty(S, dtype=torch.uint8, device=self.device),
            "src_node": torch.empty(S, dtype=torch.int32, device=self.device),
            "packed_slot": torch.empty(S, dtype=torch.int32, device=self.device),
            "slot_row": torch.empty(S, dtype=torch.int32, device=self.device),
            "packed_count": torch.zeros(1, dtype=torch.int32, device=self.device),
        })

    def load_states(self, states) -> None:
        """Copy per-layer fold states (recompute, src_node, packed_slot, slot_row,
        packed_count as host arrays) into the device buffers of layers 0, 1, ..."""
        for l, st in enumerate(states):
            self._load_state(l, st)

    def _load_state(self, l: int, st) -> None:
        dev = self.states[l]
        for k in ("recompute", "src_node", "packed_slot", "slot_row", "packed_count"):
            v = np.asarray(st[k]).reshape(-1)
            v = v.astype(np.uint8 if k == "recompute" else np.int32)
            dev[k][: v.size].copy_(torch.from_numpy(v).to(self.device))

    def forward(self, tau: float, stream=None, state_in: bool = False,
                record_states: bool = True, num_layers: Optional[int] = None) -> torch.Tensor:
        """The first num_layers layers (default: all) on H; the last one's output lands
        in self.out."""
        flags = L.SPECFOLD_FLAG_FOLD_STATE_IN if state_in else 0
        L.specfold_stack_forward(self.shape, self.w, self.prefix if self.cfg.prefix else None,
                                 self.H, self.out, self.fold_src, tau,
                                 self.states if (record_states or state_in) else None, flags,
                                 self.ws, self.ws_bytes, stream, num_layers=num_layers)
        return self.out

    def capture(self, tau: float, record_states: bool = True) -> "torch.cuda.CUDAGraph":
        """The whole stack (one specfold_stack_forward) captured as one HIP graph; replay()
        re-runs every layer's gate, packing and kernels on the current contents of H.  The
        library records no memset or allocation, only kernel launches."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward(tau, record_states=record_states)
        return g

    def layer_forward(self, l: int, x, tau: float, stream=None, state_in=None) -> torch.Tensor:
        """Layer l alone (specfold_layer_forward) on hidden state x, with the stack's
        buffers; the fold state goes to (or, given state_in, comes from) layer l's state
        buffers."""
        if not hasattr(self, "xbuf"):
            self.xbuf = torch.empty_like(self.H)
        if isinstance(x, torch.Tensor):
            self.xbuf.copy_(x.reshape(self.xbuf.shape))
        else:
            self.xbuf.copy_(to_device(np.asarray(x, dtype=np.float32).reshape(self.xbuf.shape),
                                      self.dt, self.device))
        flags = 0
        if state_in is not None:
            self._load_state(l, state_in)
            flags = L.SPECFOLD_FLAG_FOLD_STATE_IN
        L.specfold_layer_forward(self.shape, self.w[l], self.prefix[l] if self.cfg.prefix else None,
                                 self.xbuf, self.out, self.fold_src, tau, self.states[l], flags,
                                 self.ws, self.ws_bytes, stream)
        return self.out

    def fold_states(self):
        N, B = self.cfg.num_nodes, self.cfg.block
        res = []
        for dev in self.states:
            st = {k: v.cpu().numpy() for k, v in dev.items()}
            K = int(st["packed_count"][0])
            res.append(dict(ratio=st["ratio"].reshape(N, B),
                            recompute=st["recompute"].reshape(N, B) != 0,
                            src=st["src_node"].reshape(N, B), packed_slot=st["packed_slot"][:K],
                            slot_row=st["slot_row"].reshape(N, B), K=K))
        return res

    def output_numpy(self) -> np.ndarray:
        cfg = self.cfg
        return self.out.float().cpu().numpy().reshape(cfg.num_nodes, cfg.block, cfg.hidden)
