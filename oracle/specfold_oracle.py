"""CPU oracle of the folded multi-branch verify layer (SpecFold).

TEST INFRASTRUCTURE ONLY.  This module is a plain, slow, deliberately unoptimised
restatement of what one folded verify layer computes.  Only the test-suite, the
package smoke check and the benchmark's CPU-baseline leg may import it; the HIP
library never calls it and shares no code with it.

Sources (the pages are cited by title and section; no code from them is used):
  [SF]  "SpecFold" explainer, blog.ontle.kr/blog/358 -- the paragraphs on measuring the
        parent/child difference at the layer input, reusing the parent's computation,
        keeping the child's own delta, packing every branch's recompute positions into
        one batch, the shared prefix cache referenced without copies, and the
        implementation memo (gate kernel, provenance kernel, streaming attention whose
        folded outputs are corrected with the branch's own keys/values, GQA).
  [SFa] "SpecFold uskoryaet diffuzionnye yazykovye modeli do 1,99x", iitog.ru -- the
        abstract summary: token-level residual gating, folded attention and FFN that
        reuse the parent branch while keeping residual hidden states.
  [SP]  Spiffy explainer, lifetechia.com/?p=5403 -- section on the directed draft graph
        (a node may have several parents).

Precision: the layer arithmetic runs in float64 by default (``dtype`` may select
float32).  The gate ratio that decides fold-vs-recompute is also computed in float32,
the precision in which the kernels take that decision; a float64 copy is returned for
the tie band around tau.

Readings where the pages are silent (each one is listed in the design notes):
  * the ratio is measured against the fold source = the node's first parent;
  * fold iff r <= tau (so tau < 0 folds nothing and NaN recomputes); the root never folds;
  * ||parent|| = 0 gives r = 0 if the rows are equal, else +inf;
  * a folded slot takes the Q/K/V and FFN output of its *resolved* source (the ancestor
    that actually computed it);
  * attention: bidirectional inside the block, full prefix, scale 1/sqrt(dh), GQA head
    h uses KV head h // (n_q / n_kv); a folded slot's query is its source's, its keys and
    values are its own branch's block rows, so the O projection runs for every slot;
  * RMSNorm(x) = x / sqrt(mean(x^2) + eps) * g; SwiGLU FFN = (SiLU(a Wg^T) * (a Wu^T)) Wd^T;
    no biases, no rotary embedding;
  * in a stack the gate runs again at every layer on the carried residual stream; for
    bf16 models that stream is handed from layer to layer in bf16.
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "gate", "resolve", "pack", "rms_norm", "silu", "layer", "serial_layer",
    "bruteforce_provenance", "FoldState", "fold_state", "round_to_bf16", "stack",
    "lm_head_argmax", "rope",
]


# ---------------------------------------------------------------------------------------
# (1) Gate -- [SF] paragraph on measuring ||H_child - H_parent|| / ||H_parent|| at the
#     layer input; [SFa] "token-level residual gating".
# ---------------------------------------------------------------------------------------
def _ratio(c: np.ndarray, p: np.ndarray, acc) -> float:
    diff = c.astype(acc) - p.astype(acc)
    num = np.sqrt(np.sum(diff * diff, dtype=acc), dtype=acc)
    den = np.sqrt(np.sum(p.astype(acc) * p.astype(acc), dtype=acc), dtype=acc)
    if den == 0:
        return 0.0 if num == 0 else math.inf
    return acc(num / den)


def gate(H: np.ndarray, fold_src: np.ndarray, tau: float
         ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Per (node, position) relative residual and the recompute decision.

    H: [N, B, d] hidden states at the layer input; fold_src[n] = fold source of node n
    (fold_src[0] = -1).  Returns (r32 [N,B] float32, r64 [N,B] float64, recompute [N,B]
    bool).  recompute = not (r32 <= tau); root rows always recompute (r = +inf)."""
    N, B, _ = H.shape
    r32 = np.full((N, B), np.inf, dtype=np.float32)
    r64 = np.full((N, B), np.inf, dtype=np.float64)
    for n in range(1, N):
        p_node = int(fold_src[n])
        for i in range(B):
            r32[n, i] = _ratio(H[n, i], H[p_node, i], np.float32)
            r64[n, i] = _ratio(H[n, i], H[p_node, i], np.float64)
    recompute = ~(r32 <= np.float32(tau))
    recompute[0, :] = True
    return r32, r64, recompute


# ---------------------------------------------------------------------------------------
# (2) Provenance -- [SF] implementation memo: a kernel follows fold chains and links every
#     folded position to the parent state that really computed it.
# ---------------------------------------------------------------------------------------
def resolve(recompute: np.ndarray, fold_src: np.ndarray) -> np.ndarray:
    """src[n, i] = n if slot (n, i) recomputes, else src[fold_src[n], i].

    Nodes are visited in topological order (fold_src[n] < n)."""
    N, B = recompute.shape
    src = np.empty((N, B), dtype=np.int32)
    for n in range(N):
        for i in range(B):
            if recompute[n, i] or n == 0:
                src[n, i] = n
            else:
                src[n, i] = src[int(fold_src[n]), i]
    return src


def bruteforce_provenance(recompute: np.ndarray, fold_src: np.ndarray) -> np.ndarray:
    """Independent formulation of the provenance for tiny graphs: among the first-parent
    ancestors of n (n included), the recomputing one with the greatest depth, provided no
    recomputing node lies between it and n -- i.e. the nearest recomputing ancestor."""
    N, B = recompute.shape
    depth = {0: 0}
    for n in range(1, N):
        depth[n] = depth[int(fold_src[n])] + 1
    out = np.empty((N, B), dtype=np.int32)
    for n in range(N):
        chain = {n}
        m = n
        while m != 0:
            m = int(fold_src[m])
            chain.add(m)
        for i in range(B):
            cands = [a for a in chain if recompute[a, i] or a == 0]
            out[n, i] = max(cands, key=lambda a: depth[a])
    return out


# ---------------------------------------------------------------------------------------
# (3) Packing -- [SF]: recompute positions from all branches are gathered into one bundle
#     so the heavy layer runs once on it.
# ---------------------------------------------------------------------------------------
def pack(recompute: np.ndarray, src: np.ndarray
         ) -> Tuple[np.ndarray, np.ndarray, int]:
    """packed_slot = recompute slot ids (n*B + i) in ascending order; slot_row[n, i] =
    packed row of slot (src[n, i], i); K = number of packed rows."""
    N, B = recompute.shape
    packed_slot = np.flatnonzero(recompute.reshape(-1)).astype(np.int32)
    row_of = {int(s): k for k, s in enumerate(packed_slot)}
    slot_row = np.empty((N, B), dtype=np.int32)
    for n in range(N):
        for i in range(B):
            slot_row[n, i] = row_of[int(src[n, i]) * B + i]
    return packed_slot, slot_row, len(packed_slot)


class FoldState(dict):
    """recompute, src, packed_slot, slot_row, K (and the ratios when the gate ran)."""


def fold_state(H: np.ndarray, fold_src: np.ndarray, tau: float) -> FoldState:
    r32, r64, rec = gate(H, fold_src, tau)
    src = resolve(rec, fold_src)
    ps, sr, K = pack(rec, src)
    return FoldState(r32=r32, r64=r64, recompute=rec, src=src, packed_slot=ps,
                     slot_row=sr, K=K)


# ---------------------------------------------------------------------------------------
# Layer pieces (a pre-norm GQA decoder layer with a SwiGLU FFN).
# ---------------------------------------------------------------------------------------
def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def _softmax(z: np.ndarray) -> np.ndarray:
    z = z - np.max(z, axis=-1, keepdims=True)
    e = np.exp(z)
    return e / np.sum(e, axis=-1, keepdims=True)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary position embedding, rotate-half form: x [..., rows, heads, dh] at positions
    pos [rows]; element j of the first half and element j of the second half form a pair
    turned by the angle pos * theta^(-2j/dh)."""
    dh = x.shape[-1]
    half = dh // 2
    inv = np.asarray(theta, dtype=np.float64) ** (-2.0 * np.arange(half) / dh)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]          # [rows, half]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def layer(weights: Dict[str, np.ndarray], H: np.ndarray, fold_src: np.ndarray, tau: float,
          prefix_k: np.ndarray, prefix_v: np.ndarray, *, n_q: int, n_kv: int,
          eps: float = 1e-6, dtype=np.float64, state: Optional[FoldState] = None,
          slots: Optional[Iterable[Tuple[int, int]]] = None,
          attn: str = "correct", rope_theta: float = 0.0) -> Dict[str, np.ndarray]:
    """One folded verify layer over the parent and all draft branches.

    weights: rms1 [d], w_qkv [(n_q+2n_kv)dh, d] (Q heads | K heads | V heads), w_o
    [d, n_q dh], rms2 [d], w_gate_up [2ff, d] (gate rows | up rows), w_down [d, ff].
    H: [N, B, d]; prefix_k / prefix_v: [P, n_kv, dh] (P may be 0).
    state: a precomputed fold state (recompute/src/packed_slot/slot_row/K) to use
    instead of running the gate -- e.g. one taken from ``fold_state`` on other inputs.
    slots: evaluate only these (n, i) outputs (and what they depend on); other entries
    of the returned per-slot arrays are NaN.
    weights["b_qkv"] (optional): a bias added to the Q/K/V projections.
    rope_theta > 0: the Q and K heads of a packed row at block position i are rotated at
    absolute position P + i (the block follows the P prefix tokens, whose cached keys are
    stored already rotated); a folded slot's query is its source's, at the same position.
    attn: "correct" (a folded slot's attention runs against its own branch's keys and
    values -- the correction of [SF]'s implementation memo) or "reuse" (a folded slot
    takes its resolved source's attention output as it is, so only the packed rows need
    the O projection; then y[n, i] - y[src, i] = H[n, i] - H[src, i] exactly).

    Steps ([SF] paragraphs on reuse, packing and the implementation memo; [SFa]):
      1-3. gate, provenance, packing;
      4.   Q/K/V of every packed row from RMSNorm(H[packed slot]);
      5.   attention of every slot (n, i), head h: query = Q[slot_row[n,i], h], keys and
           values = the prefix followed by branch n's own block rows K/V[slot_row[n,j]];
      6.   h = H + o W_o^T for every slot;
      7.   FFN of every packed row from RMSNorm(h[packed slot]);
      8.   y[n, i] = h[n, i] + F[slot_row[n, i]]  (a folded slot keeps its own residual
           stream and adds its source's FFN output)."""
    N, B, d = H.shape
    dt = dtype
    if state is None:
        state = fold_state(H, fold_src, tau)
    rec, src = state["recompute"], state["src"]
    packed_slot, slot_row, K = state["packed_slot"], state["slot_row"], int(state["K"])

    wqkv = weights["w_qkv"].astype(dt)
    dh = wqkv.shape[0] // (n_q + 2 * n_kv)
    g = n_q // n_kv
    Hf = H.astype(dt).reshape(N * B, d)

    # (4) packed Q/K/V
    A1 = rms_norm(Hf[packed_slot], weights["rms1"].astype(dt), eps)
    qkv = A1 @ wqkv.T                                        # [K, (n_q+2n_kv) dh]
    if weights.get("b_qkv") is not None:
        qkv = qkv + weights["b_qkv"].astype(dt)
    Qp = qkv[:, : n_q * dh].reshape(K, n_q, dh)
    Kp = qkv[:, n_q * dh:(n_q + n_kv) * dh].reshape(K, n_kv, dh)
    Vp = qkv[:, (n_q + n_kv) * dh:].reshape(K, n_kv, dh)
    if rope_theta:
        pos = prefix_k.shape[0] + np.asarray(packed_slot) % B
        Qp = rope(Qp, pos, rope_theta)
        Kp = rope(Kp, pos, rope_theta)

    # which slots to evaluate
    if slots is None:
        want = np.ones((N, B), dtype=bool)
    else:
        want = np.zeros((N, B), dtype=bool)
        for (n, i) in slots:
            want[n, i] = True
    need_attn = want.copy()
    for n in range(N):
        for i in range(B):
            if want[n, i]:
                need_attn[src[n, i], i] = True

    # (5) attention per branch and head
    pk = prefix_k.astype(dt)
    pv = prefix_v.astype(dt)
    scale = 1.0 / math.sqrt(dh)
    o = np.full((N, B, n_q, dh), np.nan, dtype=dt)
    for n in range(N):
        pos = np.flatnonzero(need_attn[n])
        if len(pos) == 0:
            continue
        rows = slot_row[n]                                   # branch n's block rows
        for h in range(n_q):
            kvh = h // g
            keys = np.concatenate([pk[:, kvh], Kp[rows, kvh]], axis=0)    # [P+B, dh]
            vals = np.concatenate([pv[:, kvh], Vp[rows, kvh]], axis=0)
            q = Qp[rows[pos], h]                                          # [|pos|, dh]
            w = _softmax((q @ keys.T) * scale)
            o[n, pos, h] = w @ vals

    if attn == "reuse":
        for n in range(N):
            for i in range(B):
                if need_attn[n, i] and src[n, i] != n:
                    o[n, i] = o[src[n, i], i]
    elif attn != "correct":
        raise ValueError(f"attn must be 'correct' or 'reuse', not {attn!r}")

    # (6) O projection + residual for every evaluated slot
    wo = weights["w_o"].astype(dt)
    h_out = np.full((N, B, d), np.nan, dtype=dt)
    sel = need_attn.reshape(-1)
    h_flat = h_out.reshape(N * B, d)
    h_flat[sel] = Hf[sel] + o.reshape(N * B, n_q * dh)[sel] @ wo.T

    # (7) packed FFN on the rows some evaluated slot needs
    need_row = np.zeros(K, dtype=bool)
    need_row[slot_row[want]] = True
    ff = weights["w_down"].shape[1]
    F = np.full((K, d), np.nan, dtype=dt)
    rows = np.flatnonzero(need_row)
    if len(rows):
        A2 = rms_norm(h_flat[packed_slot[rows]], weights["rms2"].astype(dt), eps)
        wgu = weights["w_gate_up"].astype(dt)
        gate_ = A2 @ wgu[:ff].T
        up = A2 @ wgu[ff:].T
        F[rows] = (silu(gate_) * up) @ weights["w_down"].astype(dt).T

    # (8) combine
    y = np.full((N, B, d), np.nan, dtype=dt)
    wn, wi = np.nonzero(want)
    y[wn, wi] = h_out[wn, wi] + F[slot_row[wn, wi]]

    out = dict(state)
    out.update(y=y, h=h_out, o=o.reshape(N, B, n_q * dh), F=F, Q=Qp, K_=Kp, V=Vp, A1=A1)
    return out


# ---------------------------------------------------------------------------------------
# Serialised execution ([SF], appendix C as described: the authors validate the batched
# implementation by running the branches one after another).
# ---------------------------------------------------------------------------------------
def serial_layer(weights: Dict[str, np.ndarray], H: np.ndarray, fold_src: np.ndarray,
                 tau: float, prefix_k: np.ndarray, prefix_v: np.ndarray, *, n_q: int,
                 n_kv: int, eps: float = 1e-6, dtype=np.float64) -> np.ndarray:
    """Branches in topological order, no packing: a branch computes Q/K/V and its FFN
    output only at its recompute positions and inherits them from its fold source's
    per-branch caches elsewhere.  Returns y [N, B, d]."""
    N, B, d = H.shape
    dt = dtype
    r32, _, rec = gate(H, fold_src, tau)
    wqkv = weights["w_qkv"].astype(dt)
    dh = wqkv.shape[0] // (n_q + 2 * n_kv)
    g = n_q // n_kv
    wo = weights["w_o"].astype(dt)
    wgu = weights["w_gate_up"].astype(dt)
    wd = weights["w_down"].astype(dt)
    ff = wd.shape[1]
    pk, pv = prefix_k.astype(dt), prefix_v.astype(dt)
    scale = 1.0 / math.sqrt(dh)
    qkv_cache = [None] * N        # per branch: [B, (n_q+2n_kv) dh]
    f_cache = [None] * N          # per branch: [B, d]
    y = np.empty((N, B, d), dtype=dt)
    for n in range(N):
        x = H[n].astype(dt)
        qkv = np.empty((B, wqkv.shape[0]), dtype=dt)
        for i in range(B):
            if rec[n, i]:
                a = rms_norm(x[i:i + 1], weights["rms1"].astype(dt), eps)
                qkv[i] = (a @ wqkv.T)[0]
            else:
                qkv[i] = qkv_cache[int(fold_src[n])][i]
        qkv_cache[n] = qkv
        Q = qkv[:, : n_q * dh].reshape(B, n_q, dh)
        Kb = qkv[:, n_q * dh:(n_q + n_kv) * dh].reshape(B, n_kv, dh)
        Vb = qkv[:, (n_q + n_kv) * dh:].reshape(B, n_kv, dh)
        o = np.empty((B, n_q, dh), dtype=dt)
        for h in range(n_q):
            kvh = h // g
            keys = np.concatenate([pk[:, kvh], Kb[:, kvh]], axis=0)
            vals = np.concatenate([pv[:, kvh], Vb[:, kvh]], axis=0)
            o[:, h] = _softmax((Q[:, h] @ keys.T) * scale) @ vals
        hb = x + o.reshape(B, n_q * dh) @ wo.T
        Fb = np.empty((B, d), dtype=dt)
        for i in range(B):
            if rec[n, i]:
                a2 = rms_norm(hb[i:i + 1], weights["rms2"].astype(dt), eps)
                Fb[i] = ((silu(a2 @ wgu[:ff].T) * (a2 @ wgu[ff:].T)) @ wd.T)[0]
            else:
                Fb[i] = f_cache[int(fold_src[n])][i]
        f_cache[n] = Fb
        y[n] = hb + Fb
    return y


# ---------------------------------------------------------------------------------------
# Stack of layers ([SF] the paragraph on the residual ripple spreading through the layers
# and the fold decision taken per layer; reading: the gate runs again at every layer on
# the carried residual stream, so a row folded at one layer may be recomputed later).
# ---------------------------------------------------------------------------------------
def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value of every element (8 significant bits, ties to even), returned
    as float64.  x = m * 2**e with 0.5 <= |m| < 1, so m * 256 rounded to an integer keeps
    8 bits; np.rint rounds halves to even.  Covers the normal range (the values handed
    between layers are O(1)); zero, inf and NaN pass through."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(m * 256.0), e - 8)


def stack(layer_params: Iterable[Tuple[Dict[str, np.ndarray], np.ndarray, np.ndarray]],
          H: np.ndarray, fold_src: np.ndarray, tau: float, *, n_q: int, n_kv: int,
          eps: float = 1e-6, dtype=np.float64, carry: Optional[str] = None,
          states: Optional[Sequence[FoldState]] = None, keep_inputs: bool = False
          ) -> Dict[str, object]:
    """Run folded verify layers one after another on the same draft graph.

    layer_params yields (weights, prefix_k, prefix_v) for layer 0, 1, ... in order (a
    generator keeps one layer's weights in memory at a time).  Layer l takes layer l-1's
    output as its input and makes its own fold decisions on it.
    carry: None hands the output on in `dtype`; "bf16" rounds every layer's output to
    bf16 first (the residual stream stored in the model's bf16 format).
    states: per-layer fold states to use instead of each layer's gate.
    Returns dict(y=last output, states=[per-layer fold state], K=[per-layer K],
    inputs=[per-layer input] when keep_inputs)."""
    if carry not in (None, "bf16"):
        raise ValueError(f"carry must be None or 'bf16', got {carry!r}")
    x = np.asarray(H, dtype=dtype)
    got_states, Ks, inputs = [], [], []
    for l, (weights, pk, pv) in enumerate(layer_params):
        if keep_inputs:
            inputs.append(x)
        st = None if states is None else states[l]
        out = layer(weights, x, fold_src, tau, pk, pv, n_q=n_q, n_kv=n_kv, eps=eps,
                    dtype=dtype, state=st)
        got_states.append(FoldState({k: out[k] for k in
                                     ("r32", "r64", "recompute", "src", "packed_slot",
                                      "slot_row", "K") if k in out}))
        Ks.append(int(out["K"]))
        y = out["y"]
        if carry == "bf16":
            y = round_to_bf16(y).astype(dtype)
        x = y
    return dict(y=x, states=got_states, K=Ks, inputs=inputs)


# ---------------------------------------------------------------------------------------
# (10) After the last layer: LM-head logits of the final layer's packed rows and every
#      branch's predicted token at every position (the verify step compares the branches'
#      predictions; the acceptance rule itself is not on the pages).  Reading: a folded
#      slot takes the prediction of its resolved source, as it takes the source's FFN
#      output ([SF] reuse path); with every slot packed (tau < 0) each slot gets its own.
# ---------------------------------------------------------------------------------------
def lm_head_argmax(y: np.ndarray, g_final: np.ndarray, w_lm: np.ndarray, state: FoldState,
                   eps: float, rows: Optional[Sequence[int]] = None,
                   dtype=np.float64) -> Dict[str, np.ndarray]:
    """y [N, B, d] final hidden states, g_final [d] final RMSNorm gain, w_lm [V, d].

    For packed row k (slot packed_slot[k]): a_k = RMSNorm(y[slot]) * g_final, logits
    a_k . w_lm[v] for every v, row_token[k] = the first index of the maximum logit,
    row_logit[k] = that maximum.  token[n, i] = row_token[slot_row[n, i]].
    `rows` limits the evaluation to some packed rows (their row_token / row_logit /
    logits entries; token is then only returned for the slots whose row was evaluated,
    -1 elsewhere)."""
    N, B, d = y.shape
    ps = np.asarray(state["packed_slot"])
    K = int(state["K"])
    ks = np.arange(K) if rows is None else np.asarray(sorted(set(int(r) for r in rows)))
    flat = y.reshape(N * B, d).astype(dtype)
    a = rms_norm(flat[ps[ks]], np.asarray(g_final, dtype=dtype), eps)
    logits = a @ np.asarray(w_lm, dtype=dtype).T
    best = np.argmax(logits, axis=1)              # first index of the maximum
    row_token = np.full(K, -1, dtype=np.int64)
    row_logit = np.full(K, np.nan, dtype=dtype)
    row_token[ks] = best
    row_logit[ks] = logits[np.arange(len(ks)), best]
    sr = np.asarray(state["slot_row"])
    token = row_token[sr]
    return dict(row_token=row_token, row_logit=row_logit, token=token, logits=logits,
                rows=ks)
