"""CPU oracle for the single-layer MoE training hot path (dispatch, expert FFN
forward, expert FFN backward).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import or run this module.  The GPU
library never calls it, shares no code with it, and the product path fails
loudly when the HIP library is missing instead of falling back to this file.

What it computes is the plain definition of a dropless, token-choice top-K MoE
layer, written out with numpy in float64:

* routing (top-K selection and gate weights) and the four integer index
  structures named in the MoEBlaze wiki note (awesome-system-papers,
  "MoEBlaze: Breaking the Memory Wall for Efficient MoE Training on Modern
  GPUs", section "Core method", sub-section "materialisation-free token
  dispatch", data-structure table): expert_token_indices,
  expert_token_offsets, token_expert_indices, token_index_map;
* the expert FFN forward that gathers each expert's rows of x, applies the
  first MLP (SiLU, or SwiGLU as in the sub-section "SwiGLU kernel fusion +
  activation checkpoint"), the second MLP, and the gate-weighted aggregation
  back into an (L, d) output (same sub-section on dispatch, "Forward"
  paragraph; Figure 1 caption on the sciencestack page: dispatch, expert
  computation, weighted aggregation);
* the backward that scatters the (L, d) output gradient through the same
  indices, recomputes SiLU from the checkpointed first-MLP outputs and
  accumulates input and weight gradients (same sub-section, "Backward"
  paragraph, and the activation-checkpoint paragraph);
* the gradient with respect to the router logits.  The pages do not describe
  it; it is the derivative of the same forward (gates = softmax over the
  selected logits) with respect to the logits, the selection itself being
  piecewise constant.

The MoEBlaze method reaches exactly this result (it is dropless and only
changes how the work is laid out), so the oracle is the definition itself,
not the three-step GPU construction.  The one place where the oracle keeps an
(L*K, d) per-route buffer is deliberate: it is the conventional formulation
the method is measured against.

Readings taken where the pages are silent:
* W1 is the gate projection, W3 the up projection (SwiGLU only), W2 the down
  projection; layouts W1, W3: [E, d, h], W2: [E, h, d]; no biases.
* Top-K ties at the K-th place go to the lower expert id.
* Gates: softmax over the K selected logits.
* Slots of a token are ordered by ascending expert id; inside an expert's
  segment tokens are ascending; token_index_map holds the absolute row
  index into expert_token_indices.
* The gate multiplies at the aggregation; in backward the per-route output
  gradient is gate * dy.

Pins (tests that tie this file to something other than itself) are in
tests/test_oracle_*.py: pure-Python brute force on tiny shapes, a hand-worked
fixture, closed forms (K = 1, K = 2 logistic form, K = E full softmax, E = K
= 1 textbook MLP), a dense every-expert-then-mask formulation, float64
central finite differences and torch CPU autograd, plus invariants of the
index structures.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "SILU",
    "SWIGLU",
    "route",
    "build_indices",
    "ffn_forward",
    "ffn_backward",
    "router_backward",
    "route_rows_forward",
    "token_rows",
    "dw_columns",
    "router_rows",
    "checkpoint_bytes",
]

SILU = 0
SWIGLU = 1


# ---------------------------------------------------------------------------
# Routing: top-K selection and gate weights
# ---------------------------------------------------------------------------

def _select_topk(logits: np.ndarray, K: int) -> np.ndarray:
    """Experts chosen by each token: the K largest logits, ties to the lower
    expert id.  A stable sort of the negated logits keeps equal values in
    ascending expert order, so the first K columns are the selection."""
    order = np.argsort(-logits, axis=1, kind="stable")
    return order[:, :K]


def route(logits: np.ndarray, K: int):
    """Token-choice top-K routing.

    Selection follows the dropless token-choice routing the note describes
    ("Core method"; the experiments' "Accuracy" paragraph: no token is
    dropped or padded).  Returns

    * token_expert_indices [L, K] int32: each token's experts, ascending
      (the "reverse map" row of the data-structure table);
    * gates [L, K] float32: softmax over the selected logits in the same slot
      order, computed in float64 and stored as float32.
    """
    logits = np.asarray(logits, dtype=np.float32)
    L, E = logits.shape
    if not (1 <= K <= E):
        raise ValueError("need 1 <= K <= E")
    chosen = _select_topk(logits, K)
    tei = np.sort(chosen, axis=1).astype(np.int32)
    z = np.take_along_axis(logits, tei, axis=1).astype(np.float64)
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    gates = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return tei, gates


# ---------------------------------------------------------------------------
# The four index structures
# ---------------------------------------------------------------------------

def build_indices(tei: np.ndarray, E: int):
    """expert_token_indices, expert_token_offsets, token_index_map from the
    per-token expert lists (data-structure table in "Core method").

    * offsets[e] .. offsets[e+1] is expert e's interval; offsets[E] = L*K.
    * eti lists, expert by expert (ascending), the tokens routed to that
      expert (ascending).
    * tim[t, k] is the absolute position p in eti of token t's k-th route,
      so eti[tim[t, k]] == t and offsets[tei[t,k]] <= p < offsets[tei[t,k]+1].
    """
    tei = np.asarray(tei)
    L, K = tei.shape
    member = np.zeros((E, L), dtype=bool)          # member[e, t]: t routed to e
    member[tei.reshape(-1), np.repeat(np.arange(L), K)] = True
    counts = member.sum(axis=1)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    e_of, t_of = np.nonzero(member)                # row-major: e ascending, then t
    eti = t_of.astype(np.int32)
    p_of = np.arange(eti.size)
    pos = np.full((E, L), -1, dtype=np.int64)
    pos[e_of, t_of] = p_of
    tim = pos[tei, np.arange(L)[:, None]].astype(np.int32)
    return eti, offsets.astype(np.int32), tim


# ---------------------------------------------------------------------------
# Expert FFN: forward and backward (float64)
# ---------------------------------------------------------------------------

def _silu(a: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def _sigmoid(a: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def _dsilu(a: np.ndarray) -> np.ndarray:
    """d/da [a * sigmoid(a)] = s * (1 + a * (1 - s)), s = sigmoid(a)."""
    s = _sigmoid(a)
    return s * (1.0 + a * (1.0 - s))


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _glu(Ae, Be, act):
    """First-MLP activation: SiLU(A), or SiLU(A) * B for SwiGLU."""
    return _silu(Ae) if act == SILU else _silu(Ae) * Be


def ffn_forward(x, W1, W3, W2, eti, offsets, tim, gates, act):
    """Expert FFN forward with gate-weighted aggregation.

    For every expert e and route rows p in [offsets[e], offsets[e+1]):
      X = x[eti[p]]             (gather from the original (L, d) input)
      A = X W1[e],  B = X W3[e] (SwiGLU only)
      G = SiLU(A) (SiLU)  or  SiLU(A) * B (SwiGLU)
      O = G W2[e]
    then y[t] = sum_k gates[t, k] * O[tim[t, k]], k ascending.

    Returns y [L, d], A [L*K, h], B [L*K, h] or None, all float64.
    """
    x = _f64(x); W1 = _f64(W1); W3 = _f64(W3); W2 = _f64(W2)
    gates = np.asarray(gates, dtype=np.float64)
    L, d = x.shape
    E, _, h = W1.shape
    K = tim.shape[1]
    R = L * K
    A = np.zeros((R, h))
    B = np.zeros((R, h)) if act == SWIGLU else None
    O = np.zeros((R, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        X = x[eti[lo:hi]]
        A[lo:hi] = X @ W1[e]
        if act == SWIGLU:
            B[lo:hi] = X @ W3[e]
        G = _glu(A[lo:hi], None if B is None else B[lo:hi], act)
        O[lo:hi] = G @ W2[e]
    y = np.zeros((L, d))
    for k in range(K):
        y += gates[:, k:k + 1] * O[tim[:, k]]
    return y, A, B


def ffn_backward(dy, x, W1, W3, W2, eti, offsets, tim, gates, act):
    """Backward of ffn_forward for dx, dW1, dW3 (SwiGLU) and dW2.

    The (L, d) output gradient reaches route p = tim[t, k] as
    dO[p] = gates[t, k] * dy[t].  Per expert:
      dW2 = G^T dO,  dG = dO W2^T,
      SwiGLU: dA = dG * B * SiLU'(A),  dB = dG * SiLU(A)
      SiLU:   dA = dG * SiLU'(A)
      dW1 = X^T dA,  dW3 = X^T dB,  dX = dA W1^T (+ dB W3^T)
    and dx[t] = sum_k dX[tim[t, k]].  An expert with no routes gets dW = 0.

    A and B are recomputed here from x in float64 (the definition), not read
    from any checkpoint.
    """
    dy = _f64(dy); x = _f64(x); W1 = _f64(W1); W3 = _f64(W3); W2 = _f64(W2)
    gates = np.asarray(gates, dtype=np.float64)
    L, d = x.shape
    E, _, h = W1.shape
    K = tim.shape[1]
    R = L * K
    dO = np.zeros((R, d))
    for k in range(K):
        dO[tim[:, k]] = gates[:, k:k + 1] * dy
    dW1 = np.zeros((E, d, h))
    dW3 = np.zeros((E, d, h)) if act == SWIGLU else None
    dW2 = np.zeros((E, h, d))
    dXr = np.zeros((R, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        X = x[eti[lo:hi]]
        Ae = X @ W1[e]
        Be = X @ W3[e] if act == SWIGLU else None
        G = _glu(Ae, Be, act)
        dW2[e] = G.T @ dO[lo:hi]
        dG = dO[lo:hi] @ W2[e].T
        if act == SWIGLU:
            dA = dG * Be * _dsilu(Ae)
            dB = dG * _silu(Ae)
            dW1[e] = X.T @ dA
            dW3[e] = X.T @ dB
            dXr[lo:hi] = dA @ W1[e].T + dB @ W3[e].T
        else:
            dA = dG * _dsilu(Ae)
            dW1[e] = X.T @ dA
            dXr[lo:hi] = dA @ W1[e].T
    dx = np.zeros((L, d))
    for k in range(K):
        dx += dXr[tim[:, k]]
    return dx, dW1, dW3, dW2


def _softmax_backward(gates, dgate):
    """d(logit) of the selected experts from d(gate): for a softmax over the
    selected logits, dz_k = g_k * (dg_k - sum_j g_j dg_j)."""
    s = (gates * dgate).sum(axis=1, keepdims=True)
    return gates * (dgate - s)


def router_backward(dy, x, W1, W3, W2, eti, offsets, tei, tim, gates, act):
    """Gradient of <y, dy> with respect to the router logits, float64 [L, E].

    y[t] = sum_k g[t, k] O[tim[t, k]] with O = G W2[e] (the un-gated expert
    output of the route), so d<y, dy>/dg[t, k] = <dy[t], O[tim[t, k]]>; the
    gates are a softmax over the K selected logits (reading 2), whose
    backward gives the selected logits' gradient; every other logit gets 0.
    """
    dy = _f64(dy); x = _f64(x); W1 = _f64(W1); W3 = _f64(W3); W2 = _f64(W2)
    gates = np.asarray(gates, dtype=np.float64)
    L, d = x.shape
    E = W1.shape[0]
    K = tim.shape[1]
    O = np.zeros((L * K, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        X = x[eti[lo:hi]]
        Ae = X @ W1[e]
        Be = X @ W3[e] if act == SWIGLU else None
        O[lo:hi] = _glu(Ae, Be, act) @ W2[e]
    dgate = np.zeros((L, K))
    for k in range(K):
        dgate[:, k] = (dy * O[tim[:, k]]).sum(axis=1)
    dz = np.zeros((L, E))
    np.put_along_axis(dz, np.asarray(tei, dtype=np.int64), _softmax_backward(gates, dgate), axis=1)
    return dz


# ---------------------------------------------------------------------------
# Sampled evaluation for shapes too large to run whole on the host.
# Each function computes the same quantities as ffn_forward / ffn_backward /
# router_backward for a subset of outputs, with the same formulas applied to
# the subset's rows; rows that share an expert are multiplied together.
# Tests check them against the full versions.
# ---------------------------------------------------------------------------

def route_rows_forward(p_rows, x, W1, W3, eti, offsets, act):
    """A[p], B[p] (float64) for the listed route rows p: row p belongs to the
    expert whose interval of offsets holds it and reads x[eti[p]]."""
    p_rows = np.asarray(p_rows, dtype=np.int64)
    e_of = np.searchsorted(np.asarray(offsets, dtype=np.int64), p_rows, side="right") - 1
    h = W1.shape[2]
    A = np.zeros((p_rows.size, h))
    B = np.zeros((p_rows.size, h)) if act == SWIGLU else None
    for e in np.unique(e_of):
        sel = np.flatnonzero(e_of == e)
        X = _f64(x[np.asarray(eti)[p_rows[sel]]])
        A[sel] = X @ _f64(W1[e])
        if act == SWIGLU:
            B[sel] = X @ _f64(W3[e])
    return A, B


def token_rows(tokens, dy, x, W1, W3, W2, tei, tim, gates, act):
    """y[t] and dx[t] (float64) for the listed tokens.

    Every quantity of one route depends only on its own token row, so the
    rows of y and dx follow from the same formulas as ffn_forward /
    ffn_backward applied to the listed tokens' routes alone.  Slot k of each
    token is added in ascending k; the tokens whose slot-k expert is e are
    evaluated together.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    K = tei.shape[1]
    d = x.shape[1]
    X = _f64(x[tokens])
    DY = _f64(dy[tokens]) if dy is not None else None
    y = np.zeros((tokens.size, d))
    dx = np.zeros((tokens.size, d))
    for k in range(K):
        ek = np.asarray(tei)[tokens, k]
        gk = np.asarray(gates, dtype=np.float64)[tokens, k]
        for e in np.unique(ek):
            sel = np.flatnonzero(ek == e)
            g = gk[sel][:, None]
            w1, w2 = _f64(W1[e]), _f64(W2[e])
            w3 = _f64(W3[e]) if act == SWIGLU else None
            a = X[sel] @ w1
            b = X[sel] @ w3 if act == SWIGLU else None
            G = _glu(a, b, act)
            y[sel] += g * (G @ w2)
            if DY is None:
                continue
            dG = (g * DY[sel]) @ w2.T
            if act == SWIGLU:
                dA = dG * b * _dsilu(a)
                dB = dG * _silu(a)
                dx[sel] += dA @ w1.T + dB @ w3.T
            else:
                dA = dG * _dsilu(a)
                dx[sel] += dA @ w1.T
    return y, dx


def dw_columns(e, cols, dy, x, W1, W3, W2, eti, offsets, tim, tei, gates, act):
    """Selected columns of dW1[e], dW3[e] (as [d, len(cols)]) and the same
    rows of dW2[e] (as [len(cols), d]), float64.

    Column j of dA (and dB) over expert e's routes needs only column j of A,
    B and dG, so the selected columns follow from the definitions without the
    full [n_e, h] products.
    """
    cols = np.asarray(cols, dtype=np.int64)
    lo, hi = int(offsets[e]), int(offsets[e + 1])
    d = x.shape[1]
    n = hi - lo
    dW1c = np.zeros((d, cols.size))
    dW3c = np.zeros((d, cols.size)) if act == SWIGLU else None
    dW2r = np.zeros((cols.size, d))
    if n == 0:
        return dW1c, dW3c, dW2r
    toks = np.asarray(eti[lo:hi], dtype=np.int64)
    X = np.asarray(x[toks], dtype=np.float64)
    # slot of expert e in each of its tokens' lists -> gate of the route
    slot = np.argmax(np.asarray(tei[toks]) == e, axis=1)
    g = np.asarray(gates, dtype=np.float64)[toks, slot]
    dO = g[:, None] * np.asarray(dy[toks], dtype=np.float64)
    w1 = np.asarray(W1[e], dtype=np.float64)[:, cols]
    w2 = np.asarray(W2[e], dtype=np.float64)[cols, :]
    Ac = X @ w1
    Bc = X @ np.asarray(W3[e], dtype=np.float64)[:, cols] if act == SWIGLU else None
    Gc = _glu(Ac, Bc, act)
    dW2r[:] = Gc.T @ dO
    dGc = dO @ w2.T
    if act == SWIGLU:
        dAc = dGc * Bc * _dsilu(Ac)
        dBc = dGc * _silu(Ac)
        dW1c[:] = X.T @ dAc
        dW3c[:] = X.T @ dBc
    else:
        dAc = dGc * _dsilu(Ac)
        dW1c[:] = X.T @ dAc
    return dW1c, dW3c, dW2r


def router_rows(tokens, dy, x, W1, W3, W2, tei, gates, act, E):
    """Rows of router_backward (float64 [len(tokens), E]) for the listed
    tokens: a token's logit gradient needs only its own K routes, evaluated
    slot by slot, the tokens that share the slot's expert together."""
    tokens = np.asarray(tokens, dtype=np.int64)
    K = tei.shape[1]
    X = _f64(x[tokens])
    DY = _f64(dy[tokens])
    dg = np.zeros((tokens.size, K))
    for k in range(K):
        ek = np.asarray(tei)[tokens, k]
        for e in np.unique(ek):
            sel = np.flatnonzero(ek == e)
            a = X[sel] @ _f64(W1[e])
            b = X[sel] @ _f64(W3[e]) if act == SWIGLU else None
            O = _glu(a, b, act) @ _f64(W2[e])
            dg[sel, k] = (DY[sel] * O).sum(axis=1)
    g = np.asarray(gates, dtype=np.float64)[tokens]
    dz = np.zeros((tokens.size, E))
    np.put_along_axis(dz, np.asarray(tei, dtype=np.int64)[tokens], _softmax_backward(g, dg),
                      axis=1)
    return dz


def checkpoint_bytes(L, K, h, act, elem_bytes):
    """Bytes of the first-MLP checkpoint kept for backward: A (and B for
    SwiGLU), one row of h per route ("SwiGLU kernel fusion + activation
    checkpoint": only A and B are kept)."""
    return L * K * h * (2 if act == SWIGLU else 1) * elem_bytes
