"""Oracle MoE layer: a plain, slow, fp64 CPU implementation.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the GPU path and
imports nothing from it: it receives the same input bits and decodes them
itself (bf16 patterns shifted into fp32, E4M3 through its own table).

What the layer computes.  The pages state the problem only in words: each
MoE layer routes every token to a few experts (dzen.guru page, "Что именно
тормозило обучение MoE-моделей?"), the expert math runs per expert (the
"expert-centric" scheme of the warp-decode page, toolnavs.com, section
"Cursor a réécrit le décodage de MoE"), and the results are gathered back in
a deterministic way (dzen.guru, megakernel paragraph of "Три решения…").
The workload recipe fixes the arithmetic, y = sum_k g_k E_k(x):

  router   l = W_r x (+ b);  p = softmax_E(l);  S = top-k of l;  g = p_S / sum_S p
  expert   E_e(x) = W_down[e] (silu(W_gate[e] x) * (W_up[e] x)),  silu(a) = a sigmoid(a)
  combine  y = sum over the k selected experts, ascending expert id, of g E_e(x)

Dispatch follows the fixed token ring buffer of the dzen.guru page (paragraph
on the ring buffer in "Три решения…"): no token is dropped, copies are laid
out expert-contiguously from a ring head, slots wrap modulo the capacity.

Readings where the pages are silent:
  * topk_idx is reported in ascending expert id; ties in l go to the lower id;
  * copies (t, j), c = t*k + j, are ordered stably by expert, i.e. by (e, t);
  * a segment occupies slots (head + offset[e] + i) mod C;
  * the shared expert of the decode workload has weight 1 outside the softmax;
  * MX: x, W_gate, W_up along d, and H, W_down along f, per 32 elements;
  * the backward holds S fixed (top-k is not differentiated); b has no gradient.

Everything is fp64; nothing is rounded back to bf16.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

from . import mx

# --------------------------------------------------------------------------- inputs


def from_bf16_bits(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64: the pattern is the top half of an fp32."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def from_f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (round to nearest even) -> bf16 (round to nearest even on the top 16
    bits), as fp64: how the forward keeps its saved pre-activations."""
    u = np.asarray(a, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return from_bf16_bits(r)


# Expert weights are handed over lazily, one expert at a time: a callable
# e -> (W_gate[e] [f,d], W_up[e] [f,d], W_down[e] [d,f]) in fp64.
Weights = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]


def weights_from_arrays(wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> Weights:
    return lambda e: (wg[e], wu[e], wd[e])


# --------------------------------------------------------------------------- O1 router


@dataclass
class Routing:
    idx: np.ndarray      # [T, k] int64, ascending expert id per token
    gate: np.ndarray     # [T, k] fp64, renormalised over the selected set
    count: np.ndarray    # [E] int64
    logits: np.ndarray   # [T, E]
    probs: np.ndarray    # [T, E]


def softmax_rows(l: np.ndarray) -> np.ndarray:
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def route(x: np.ndarray, w_r: np.ndarray, b: Optional[np.ndarray], k: int) -> Routing:
    """Router: logits, softmax over all E, top-k, renormalised gates, expert counts."""
    l = x @ w_r.T
    if b is not None:
        l = l + b[None, :]
    p = softmax_rows(l)
    order = np.argsort(-l, axis=1, kind="stable")      # descending, ties to the lower id
    S = np.sort(order[:, :k], axis=1)
    pS = np.take_along_axis(p, S, axis=1)
    g = pS / pS.sum(axis=1, keepdims=True)
    count = np.bincount(S.ravel(), minlength=w_r.shape[0]).astype(np.int64)
    return Routing(S.astype(np.int64), g, count, l, p)


# --------------------------------------------------------------------------- O2 dispatch


@dataclass
class Dispatch:
    copy_slot: np.ndarray    # [T, k] absolute ring slot of copy (t, j)
    slot_copy: np.ndarray    # [C] copy id t*k+j held by each slot, -1 where unused
    offset: np.ndarray       # [E+1] segment starts relative to the head
    head: int
    C: int


def dispatch(idx: np.ndarray, E: int, C: int, head: int = 0) -> Dispatch:
    """Stable counting sort of the copies by expert into the ring."""
    T, k = idx.shape
    n = T * k
    if C < n:
        raise ValueError("ring capacity below the number of token copies")
    keys = idx.reshape(-1)
    perm = np.argsort(keys, kind="stable")              # copy ids in ring order
    rank = np.empty(n, dtype=np.int64)
    rank[perm] = np.arange(n)
    slot = (head + rank) % C
    count = np.bincount(keys, minlength=E)
    offset = np.concatenate([[0], np.cumsum(count)]).astype(np.int64)
    slot_copy = np.full(C, -1, dtype=np.int64)
    slot_copy[slot] = np.arange(n)
    return Dispatch(slot.reshape(T, k), slot_copy, offset, head, C)


def ring_fill(rows: np.ndarray, disp: Dispatch) -> np.ndarray:
    """ring[copy_slot[t, j]] = rows[t]; unused slots are zero."""
    T, k = disp.copy_slot.shape
    ring = np.zeros((disp.C,) + rows.shape[1:], dtype=rows.dtype)
    ring[disp.copy_slot.reshape(-1)] = np.repeat(rows, k, axis=0)
    return ring


def segment_slots(disp: Dispatch, e: int) -> np.ndarray:
    """Ring slots of expert e's segment, in segment order."""
    start, stop = disp.offset[e], disp.offset[e + 1]
    return (disp.head + np.arange(start, stop)) % disp.C


# --------------------------------------------------------------------------- O3 expert FFN


def sigmoid(a: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-a))


def swiglu(X: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
           h_mx: bool = False) -> np.ndarray:
    """E(X) = W_down (silu(W_gate X) * W_up X) for a block of rows X [n, d]."""
    A = X @ wg.T
    U = X @ wu.T
    H = A * sigmoid(A) * U
    if h_mx:
        H = mx.fake_quant(H, axis=1)
    return H @ wd.T


def expert_ffn(ring: np.ndarray, disp: Dispatch, weights: Weights,
               experts: Optional[Iterable[int]] = None, h_mx: bool = False) -> np.ndarray:
    """ring_y: each expert applied to its own segment of ring rows (others stay zero)."""
    E = disp.offset.size - 1
    d_out = None
    out: Dict[int, np.ndarray] = {}
    for e in (range(E) if experts is None else experts):
        slots = segment_slots(disp, e)
        if slots.size == 0:
            continue
        wg, wu, wd = weights(e)
        out[e] = swiglu(ring[slots], wg, wu, wd, h_mx)
        d_out = out[e].shape[1]
    ring_y = np.zeros((disp.C, d_out if d_out is not None else ring.shape[1]))
    for e, y in out.items():
        ring_y[segment_slots(disp, e)] = y
    return ring_y


# --------------------------------------------------------------------------- O4 combine


def combine(ring_y: np.ndarray, copy_slot: np.ndarray, gate: np.ndarray) -> np.ndarray:
    """y[t] = sum_j gate[t, j] ring_y[copy_slot[t, j]], j in ascending expert order."""
    T, k = copy_slot.shape
    y = np.zeros((T, ring_y.shape[1]))
    for j in range(k):
        y += gate[:, j, None] * ring_y[copy_slot[:, j]]
    return y


# --------------------------------------------------------------------------- whole layer


@dataclass
class Forward:
    routing: Routing
    disp: Dispatch
    ring_x: np.ndarray
    ring_y: np.ndarray
    y: np.ndarray


def forward(x: np.ndarray, w_r: np.ndarray, b: Optional[np.ndarray], k: int,
            weights: Weights, C: int, head: int = 0, mx_path: bool = False,
            shared: Optional[Tuple[np.ndarray, np.ndarray, np.ndarray]] = None) -> Forward:
    """The layer, step by step: route, dispatch into the ring, expert FFN, combine.

    mx_path: the dispatched x and the expert weights are MX-quantised (the
    caller passes weights already decoded from their MX codes), and so is H.
    shared: an always-on expert (W_gate, W_up, W_down) added with weight 1."""
    E = w_r.shape[0]
    r = route(x, w_r, b, k)
    disp = dispatch(r.idx, E, C, head)
    rows = mx.fake_quant(x, axis=1) if mx_path else x
    ring_x = ring_fill(rows, disp)
    ring_y = expert_ffn(ring_x, disp, weights, h_mx=mx_path)
    y = combine(ring_y, disp.copy_slot, r.gate)
    if shared is not None:
        y = y + swiglu(x, *shared)
    return Forward(r, disp, ring_x, ring_y, y)


def forward_tokens(tokens: Sequence[int], x: np.ndarray, routing: Routing, weights: Weights,
                   mx_path: bool = False,
                   shared: Optional[Tuple[np.ndarray, np.ndarray, np.ndarray]] = None) -> np.ndarray:
    """y for a few tokens: y_t = sum_j g_tj E_{S_tj}(x_t) (+ shared), evaluated per token.
    The experts are visited in ascending id (each token's terms in its j order), so that a
    lazy weight accessor loads every expert once."""
    tokens = np.asarray(tokens, dtype=np.int64)
    k = routing.idx.shape[1]
    xs = x[tokens]
    xq = mx.fake_quant(xs, axis=1) if mx_path else xs
    y = np.zeros((tokens.size, x.shape[1]))
    for e in np.unique(routing.idx[tokens]):
        wg, wu, wd = weights(int(e))
        for i, t in enumerate(tokens):
            for j in range(k):
                if routing.idx[t, j] == e:
                    y[i] += routing.gate[t, j] * swiglu(xq[i:i + 1], wg, wu, wd, h_mx=mx_path)[0]
    if shared is not None:
        y += swiglu(xs, *shared)
    return y


# --------------------------------------------------------------------------- brute force


def brute_force(x: np.ndarray, w_r: np.ndarray, b: Optional[np.ndarray], k: int,
                weights: Weights,
                shared: Optional[Tuple[np.ndarray, np.ndarray, np.ndarray]] = None) -> np.ndarray:
    """Per-token loop, every expert evaluated densely, no sort, no segment, no ring.
    Only for tiny shapes.  shared: an always-on expert (W_gate, W_up, W_down) whose
    output joins every token's sum with weight 1, outside the softmax."""
    T, _ = x.shape
    E = w_r.shape[0]
    y = np.zeros_like(x)
    for t in range(T):
        if shared is not None:
            sg, su, sd = shared
            hs = []
            for i in range(sg.shape[0]):
                a_i = float(np.dot(sg[i], x[t]))
                hs.append(a_i / (1.0 + np.exp(-a_i)) * float(np.dot(su[i], x[t])))
            y[t] += sd @ np.array(hs)
        lt = [float(np.dot(w_r[e], x[t])) + (0.0 if b is None else float(b[e])) for e in range(E)]
        outs = []
        for e in range(E):
            wg, wu, wd = weights(e)
            a = wg @ x[t]
            u = wu @ x[t]
            h = [a[i] / (1.0 + np.exp(-a[i])) * u[i] for i in range(a.size)]
            outs.append(wd @ np.array(h))
        # pick k experts by repeated max (first index wins a tie)
        chosen = []
        for _ in range(k):
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or lt[e] > lt[best]:
                    best = e
            chosen.append(best)
        m = max(lt)
        w = {e: np.exp(lt[e] - m) for e in chosen}
        z = sum(w.values())
        for e in sorted(chosen):
            y[t] += (w[e] / z) * outs[e]
    return y


# --------------------------------------------------------------------------- O5 backward


@dataclass
class ExpertGrad:
    dw_gate: np.ndarray   # [f, d]
    dw_up: np.ndarray     # [f, d]
    dw_down: np.ndarray   # [d, f]
    tokens: np.ndarray    # [n_e] token ids of the expert's copies (ascending)
    js: np.ndarray        # [n_e] position j of the expert in each token's top-k
    dg: np.ndarray        # [n_e] dL/dg for each copy
    dx: np.ndarray        # [n_e, d] expert-path input gradient of each copy


def expert_backward(e: int, x: np.ndarray, dy: np.ndarray, routing: Routing,
                    weights: Weights) -> ExpertGrad:
    """Gradients of L = sum_t <dy_t, y_t> through expert e, S held fixed.

    For a copy (t, j) of expert e with gate g:
      a = W_g x, u = W_u x, s = sigmoid(a), h = a s u
      dh_raw = W_d^T dy,  dg = <dh_raw, h>,  dh = g dh_raw
      da = dh u s (1 + a (1 - s)),  du = dh a s
      dx_c = W_g^T da + W_u^T du
      dW_d += g dy h^T,  dW_g += da x^T,  dW_u += du x^T
    """
    ts, js = np.nonzero(routing.idx == e)
    wg, wu, wd = weights(e)
    f, d = wg.shape
    if ts.size == 0:
        z = np.zeros
        return ExpertGrad(z((f, d)), z((f, d)), z((d, f)), ts, js, z(0), z((0, d)))
    X = x[ts]
    g = routing.gate[ts, js]
    A = X @ wg.T
    U = X @ wu.T
    s = sigmoid(A)
    H = A * s * U
    dHraw = dy[ts] @ wd
    dg = np.sum(dHraw * H, axis=1)
    dH = g[:, None] * dHraw
    dA = dH * U * s * (1.0 + A * (1.0 - s))
    dU = dH * A * s
    dxc = dA @ wg + dU @ wu
    return ExpertGrad(dA.T @ X, dU.T @ X, (g[:, None] * dy[ts]).T @ H, ts, js, dg, dxc)


@dataclass
class Backward:
    dx: np.ndarray
    dw_gate: np.ndarray
    dw_up: np.ndarray
    dw_down: np.ndarray
    dw_router: np.ndarray
    dg: np.ndarray        # [T, k]
    dl: np.ndarray        # [T, k] logit gradients on the selected set


def router_logit_grad(gate: np.ndarray, dg: np.ndarray) -> np.ndarray:
    """g = softmax over the selected logits, so dl_j = g_j (dg_j - sum_i g_i dg_i)."""
    return gate * (dg - np.sum(gate * dg, axis=1, keepdims=True))


def backward(x: np.ndarray, w_r: np.ndarray, routing: Routing, weights: Weights,
             dy: np.ndarray) -> Backward:
    """Full backward of L = sum_t <dy_t, y_t> (S fixed, b a constant)."""
    T, d = x.shape
    E, k = w_r.shape[0], routing.idx.shape[1]
    dx = np.zeros((T, d))
    dg = np.zeros((T, k))
    grads = []
    for e in range(E):
        eg = expert_backward(e, x, dy, routing, weights)
        grads.append(eg)
        dg[eg.tokens, eg.js] = eg.dg
        np.add.at(dx, eg.tokens, eg.dx)
    dl = router_logit_grad(routing.gate, dg)
    dw_r = np.zeros((E, d))
    for j in range(k):
        np.add.at(dw_r, routing.idx[:, j], dl[:, j, None] * x)
        dx += dl[:, j, None] * w_r[routing.idx[:, j]]
    return Backward(dx, np.stack([g.dw_gate for g in grads]), np.stack([g.dw_up for g in grads]),
                    np.stack([g.dw_down for g in grads]), dw_r, dg, dl)


def backward_tokens(tokens: Sequence[int], x: np.ndarray, w_r: np.ndarray, routing: Routing,
                    weights: Weights, dy: np.ndarray):
    """dx, dg and dl of a few tokens, each computed from that token's k copies only."""
    tokens = np.asarray(tokens, dtype=np.int64)
    k = routing.idx.shape[1]
    dx = np.zeros((tokens.size, x.shape[1]))
    dg = np.zeros((tokens.size, k))
    for i, t in enumerate(tokens):
        for j in range(k):
            e = int(routing.idx[t, j])
            wg, wu, wd = weights(e)
            a = wg @ x[t]
            u = wu @ x[t]
            s = sigmoid(a)
            h = a * s * u
            dhr = wd.T @ dy[t]
            dg[i, j] = dhr @ h
            dh = routing.gate[t, j] * dhr
            da = dh * u * s * (1.0 + a * (1.0 - s))
            du = dh * a * s
            dx[i] += wg.T @ da + wu.T @ du
    dl = router_logit_grad(routing.gate[tokens], dg)
    for j in range(k):
        dx += dl[:, j, None] * w_r[routing.idx[tokens, j]]
    return dx, dg, dl


def router_weight_grad_rows(experts: Sequence[int], x: np.ndarray, w_r: np.ndarray,
                            routing: Routing, weights: Weights, dy: np.ndarray) -> np.ndarray:
    """Rows of dW_r for a few experts: sum over the tokens that selected e of dl[t, e] x_t."""
    out = np.zeros((len(experts), x.shape[1]))
    for i, e in enumerate(experts):
        ts, js = np.nonzero(routing.idx == e)
        if ts.size == 0:
            continue
        _, _, dl = backward_tokens(ts, x, w_r, routing, weights, dy)
        out[i] = (dl[np.arange(ts.size), js][:, None] * x[ts]).sum(axis=0)
    return out


# --------------------------------------------------------------------------- metric


def max_abs_rel(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| over one tensor."""
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    err = np.max(np.abs(np.asarray(got, dtype=np.float64) - ref)) if ref.size else 0.0
    return float(err / den) if den > 0 else float(err)


# --------------------------------------------------------------------------- O6 MXFP8 backward
#
# The pages report the layer's MXFP8 backward (dzen.guru page, "Что показали замеры?") without
# its recipe.  Reading: each backward GEMM takes its two operands MX-quantised (E4M3, one E8M0
# scale per 32) along that GEMM's own reduction dimension, products accumulated exactly (fp64
# here), everything elementwise unquantised; the forward's quantisation is the identity in
# the backward (straight-through), and A, U are the MX forward's as the forward saves them,
# rounded to bf16 (each backward GEMM re-quantises values derived from them, so a rounding
# there moves values across E4M3 rounding boundaries and is part of the definition):
#   A = bf16(Q_d(X) Q_d(W_gate)^T),  U = bf16(Q_d(X) Q_d(W_up)^T),  H = silu(A) U
#   dH_raw = Q_d(dY) Q_d(W_down)          W_down [d, f] quantised along d (its columns)
#   dg = <dH_raw, H>;  dA, dU as in the bf16 backward
#   dX_c = Q_f(dA) Q_f(W_gate) + Q_f(dU) Q_f(W_up)     W_gate, W_up [f, d] along f
#   dW_down = Q_t(dY)^T Q_t(g H),  dW_gate = Q_t(dA)^T Q_t(X),  dW_up = Q_t(dU)^T Q_t(X)
# Q_t quantises along the token axis: an expert's copies in ring-segment order (ascending
# token), in blocks of 32 aligned to the segment's end (the first block is the partial one:
# the backward walks the ring last slot first).  The router part is the bf16 backward's.


def token_quant(M: np.ndarray) -> np.ndarray:
    """MX round trip of the rows of M (an expert's copies in segment order) along the row
    axis, blocks of 32 rows aligned to the last row (zero rows pad the first block)."""
    n = M.shape[0]
    pad = (-n) % mx.BLOCK
    P = np.concatenate([np.zeros((pad,) + M.shape[1:]), M], axis=0)
    return mx.fake_quant(P, axis=0)[pad:]


def expert_backward_mx(e: int, x: np.ndarray, dy: np.ndarray, routing: Routing,
                       weights: Weights, disp: Dispatch) -> ExpertGrad:
    """Gradients through expert e in the MXFP8 layer (weights: the bf16 weights in fp64)."""
    k = routing.idx.shape[1]
    copies = disp.slot_copy[segment_slots(disp, e)]      # ring-segment order
    ts, js = copies // k, copies % k
    wg, wu, wd = weights(e)
    f, d = wg.shape
    if ts.size == 0:
        z = np.zeros
        return ExpertGrad(z((f, d)), z((f, d)), z((d, f)), ts, js, z(0), z((0, d)))
    X = x[ts]
    g = routing.gate[ts, js]
    Xq = mx.fake_quant(X, axis=1)
    A = round_bf16(Xq @ mx.fake_quant(wg, axis=1).T)
    U = round_bf16(Xq @ mx.fake_quant(wu, axis=1).T)
    s = sigmoid(A)
    H = A * s * U
    dY = dy[ts]
    dHraw = mx.fake_quant(dY, axis=1) @ mx.fake_quant(wd, axis=0)
    dg = np.sum(dHraw * H, axis=1)
    dH = g[:, None] * dHraw
    dA = dH * U * s * (1.0 + A * (1.0 - s))
    dU = dH * A * s
    dxc = (mx.fake_quant(dA, axis=1) @ mx.fake_quant(wg, axis=0)
           + mx.fake_quant(dU, axis=1) @ mx.fake_quant(wu, axis=0))
    Xt = token_quant(X)
    return ExpertGrad(token_quant(dA).T @ Xt, token_quant(dU).T @ Xt,
                      token_quant(dY).T @ token_quant(g[:, None] * H), ts, js, dg, dxc)


def backward_mx(x: np.ndarray, w_r: np.ndarray, routing: Routing, weights: Weights,
                dy: np.ndarray, disp: Dispatch) -> Backward:
    """The MXFP8 layer's backward of L = sum_t <dy_t, y_t> (S fixed, b a constant)."""
    T, d = x.shape
    E, k = w_r.shape[0], routing.idx.shape[1]
    dx = np.zeros((T, d))
    dg = np.zeros((T, k))
    grads = []
    for e in range(E):
        eg = expert_backward_mx(e, x, dy, routing, weights, disp)
        grads.append(eg)
        dg[eg.tokens, eg.js] = eg.dg
        np.add.at(dx, eg.tokens, eg.dx)
    dl = router_logit_grad(routing.gate, dg)
    dw_r = np.zeros((E, d))
    for j in range(k):
        np.add.at(dw_r, routing.idx[:, j], dl[:, j, None] * x)
        dx += dl[:, j, None] * w_r[routing.idx[:, j]]
    return Backward(dx, np.stack([g.dw_gate for g in grads]), np.stack([g.dw_up for g in grads]),
                    np.stack([g.dw_down for g in grads]), dw_r, dg, dl)
