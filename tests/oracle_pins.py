"""Pins that tie the CPU oracle to something other than itself.

Each check takes an oracle module (the real one, or a copy with a planted
mistake) and raises AssertionError when the oracle disagrees with:

* a hand-worked fixture (tests/golden/dispatch_hand_example.json),
* a pure-Python brute force of selection and the index structures,
* invariants of the four index structures,
* closed forms of the gates (K = 1; K = 2 logistic form; K = E full softmax
  from scipy),
* a dense "every expert on every token, then mask" formulation in torch
  float64, differentiated by torch autograd (library routine, CPU only),
* the E = K = 1 case, which is a plain two-layer MLP (torch's SiLU),
* float64 central finite differences of <y, dy>,
* consistency of the sampled evaluators with the full forward/backward;
* for the router-logit gradient: torch autograd of the dense formulation with
  respect to the logits, float64 central finite differences of <y, dy> along
  logit directions that keep the selection, the K = 1 case (gates are 1, so
  the gradient is exactly 0) and the zero row sum of a softmax Jacobian.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SILU, SWIGLU = 0, 1


# ---------------------------------------------------------------------------
# small deterministic inputs
# ---------------------------------------------------------------------------

def tiny_inputs(L, d, h, E, K, act, seed, int_logits=False):
    rng = np.random.default_rng(seed)
    if int_logits:
        logits = rng.integers(-2, 3, size=(L, E)).astype(np.float32)
    else:
        logits = rng.standard_normal((L, E)).astype(np.float32)
    x = rng.standard_normal((L, d))
    W1 = rng.standard_normal((E, d, h)) / math.sqrt(d)
    W3 = rng.standard_normal((E, d, h)) / math.sqrt(d) if act == SWIGLU else None
    W2 = rng.standard_normal((E, h, d)) / math.sqrt(h)
    dy = rng.standard_normal((L, d))
    return logits, x, W1, W3, W2, dy


# ---------------------------------------------------------------------------
# brute force references
# ---------------------------------------------------------------------------

def brute_select(logits, K):
    """Selection by repeated arg-max over the not-yet-chosen experts, strict
    comparison scanning ascending expert ids (so ties keep the lower id)."""
    L, E = len(logits), len(logits[0])
    sel = []
    for t in range(L):
        chosen = []
        for _ in range(K):
            best = None
            for e in range(E):
                if e in chosen:
                    continue
                if best is None or logits[t][e] > logits[t][best]:
                    best = e
            chosen.append(best)
        sel.append(sorted(chosen))
    return sel


def brute_indices(logits, K):
    E = len(logits[0])
    sel = brute_select(logits, K)
    L = len(sel)
    eti, offsets = [], [0]
    for e in range(E):
        for t in range(L):
            if e in sel[t]:
                eti.append(t)
        offsets.append(len(eti))
    tim = [[None] * K for _ in range(L)]
    for e in range(E):
        for p in range(offsets[e], offsets[e + 1]):
            t = eti[p]
            tim[t][sel[t].index(e)] = p
    return sel, eti, offsets, tim


def rank_mask(Z, K):
    """mask[t, e] = e is among the K largest of row t (ties: lower id first),
    computed by counting for each e how many experts beat it."""
    L, E = Z.shape
    j = torch.arange(E)
    beats = Z[:, None, :] > Z[:, :, None]                   # [t, e, j]: j beats e
    ties_lower = (Z[:, None, :] == Z[:, :, None]) & (j[None, None, :] < j[None, :, None])
    rank = beats.sum(-1) + ties_lower.sum(-1)
    return rank < K


def dense_mask_torch(logits, x, W1, W3, W2, dy, K, act):
    """Dense formulation: every expert on every token, weighted by a gate that
    is zero for unselected experts; gradients by torch autograd (float64)."""
    Z = torch.tensor(np.asarray(logits, dtype=np.float64), requires_grad=True)
    mask = rank_mask(Z.detach(), K)
    gate = torch.softmax(torch.where(mask, Z, torch.full_like(Z, -math.inf)), dim=1)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    w1 = torch.tensor(W1, dtype=torch.float64, requires_grad=True)
    w2 = torch.tensor(W2, dtype=torch.float64, requires_grad=True)
    w3 = torch.tensor(W3, dtype=torch.float64, requires_grad=True) if act == SWIGLU else None
    y = torch.zeros(x.shape, dtype=torch.float64)
    for e in range(W1.shape[0]):
        a = xt @ w1[e]
        G = F.silu(a) * (xt @ w3[e]) if act == SWIGLU else F.silu(a)
        y = y + gate[:, e:e + 1] * (G @ w2[e])
    (y * torch.tensor(dy, dtype=torch.float64)).sum().backward()
    out = dict(y=y.detach().numpy(), dx=xt.grad.numpy(), dW1=w1.grad.numpy(),
               dW2=w2.grad.numpy(), dW3=None if w3 is None else w3.grad.numpy(),
               dlogits=Z.grad.numpy(), mask=mask.numpy(), gate=gate.detach().numpy())
    return out


def relerr(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


# ---------------------------------------------------------------------------
# checks
# ---------------------------------------------------------------------------

def check_golden_dispatch(orc):
    with open(os.path.join(GOLDEN, "dispatch_hand_example.json")) as f:
        g = json.load(f)
    logits = np.array(g["logits"], dtype=np.float32)
    tei, gates = orc.route(logits, g["K"])
    eti, offsets, tim = orc.build_indices(tei, g["E"])
    assert tei.tolist() == g["token_expert_indices"], tei.tolist()
    assert offsets.tolist() == g["expert_token_offsets"], offsets.tolist()
    assert eti.tolist() == g["expert_token_indices"], eti.tolist()
    assert tim.tolist() == g["token_index_map"], tim.tolist()
    assert np.allclose(gates, np.array(g["gates"]), rtol=0, atol=1e-7), gates


def check_bruteforce_indices(orc):
    cases = [(1, 1, 1, False), (7, 3, 1, False), (19, 5, 2, True), (33, 6, 3, True),
             (24, 4, 4, True), (40, 8, 2, False), (12, 9, 5, True)]
    for i, (L, E, K, ints) in enumerate(cases):
        rng = np.random.default_rng(100 + i)
        if ints:
            logits = rng.integers(-1, 2, size=(L, E)).astype(np.float32)
        else:
            logits = rng.standard_normal((L, E)).astype(np.float32)
        sel, beti, boff, btim = brute_indices(logits.tolist(), K)
        tei, gates = orc.route(logits, K)
        eti, offsets, tim = orc.build_indices(tei, E)
        assert tei.tolist() == sel, (L, E, K)
        assert eti.tolist() == beti, (L, E, K)
        assert offsets.tolist() == boff, (L, E, K)
        assert tim.tolist() == btim, (L, E, K)
        assert tei.dtype == np.int32 and eti.dtype == np.int32
        assert tim.dtype == np.int32 and offsets.dtype == np.int32


def check_invariants(orc):
    for i, (L, E, K) in enumerate([(300, 8, 2), (257, 16, 4), (64, 64, 6), (129, 3, 3)]):
        rng = np.random.default_rng(7 + i)
        logits = rng.standard_normal((L, E)).astype(np.float32)
        tei, gates = orc.route(logits, K)
        eti, off, tim = orc.build_indices(tei, E)
        R = L * K
        assert off[0] == 0 and off[E] == R
        assert np.all(np.diff(off) >= 0)
        assert np.all(np.diff(tei, axis=1) > 0)                   # ascending, distinct
        assert np.array_equal(np.bincount(eti, minlength=L), np.full(L, K))
        assert np.array_equal(eti[tim], np.repeat(np.arange(L)[:, None], K, axis=1))
        lo = off[tei]
        hi = off[tei + 1]
        assert np.all((lo <= tim) & (tim < hi))
        assert np.array_equal(np.sort(tim.reshape(-1)), np.arange(R))
        for e in range(E):                                          # ascending tokens
            assert np.all(np.diff(eti[off[e]:off[e + 1]]) > 0)


def check_special_cases_indices(orc):
    rng = np.random.default_rng(3)
    L = 50
    # E = 1: every token on the only expert, identity list
    logits = rng.standard_normal((L, 1)).astype(np.float32)
    tei, gates = orc.route(logits, 1)
    eti, off, tim = orc.build_indices(tei, 1)
    assert eti.tolist() == list(range(L)) and off.tolist() == [0, L]
    assert tim[:, 0].tolist() == list(range(L)) and np.all(gates == 1.0)
    # K = E: every segment holds every token, tim[t, k] = k * L + t
    E = 5
    logits = rng.standard_normal((L, E)).astype(np.float32)
    tei, gates = orc.route(logits, E)
    eti, off, tim = orc.build_indices(tei, E)
    assert off.tolist() == [k * L for k in range(E + 1)]
    assert eti.tolist() == list(range(L)) * E
    assert np.array_equal(tim, np.arange(E)[None, :] * L + np.arange(L)[:, None])
    # full softmax over all experts (scipy)
    ref = scipy.special.softmax(logits.astype(np.float64), axis=1)
    assert np.allclose(gates, ref, rtol=0, atol=2e-7)
    # all tokens forced to one expert by a bias
    logits = rng.standard_normal((L, 6)).astype(np.float32)
    logits[:, 4] += 100.0
    tei, gates = orc.route(logits, 1)
    eti, off, tim = orc.build_indices(tei, 6)
    assert off.tolist() == [0, 0, 0, 0, 0, L, L]
    assert eti.tolist() == list(range(L))


def check_gates_closed_forms(orc):
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((200, 7)).astype(np.float32)
    _, g1 = orc.route(logits, 1)
    assert np.all(g1 == 1.0)
    tei, g2 = orc.route(logits, 2)
    z = np.take_along_axis(logits, tei, axis=1).astype(np.float64)
    logistic = scipy.special.expit(z[:, 0] - z[:, 1])
    assert np.allclose(g2[:, 0], logistic, rtol=0, atol=1e-7)
    assert np.allclose(g2[:, 1], 1.0 - logistic, rtol=0, atol=1e-7)
    for K in (3, 5):
        _, g = orc.route(logits, K)
        assert np.allclose(g.astype(np.float64).sum(1), 1.0, rtol=0, atol=1e-6)
        assert np.all(g > 0)
    # shifting a token's logits by a constant changes nothing
    tei_a, ga = orc.route(logits, 3)
    tei_b, gb = orc.route(logits + np.float32(8.0), 3)
    assert np.array_equal(tei_a, tei_b)
    assert np.allclose(ga, gb, rtol=0, atol=1e-6)


def _run_oracle(orc, logits, x, W1, W3, W2, dy, K, act):
    E = W1.shape[0]
    tei, gates = orc.route(logits, K)
    eti, off, tim = orc.build_indices(tei, E)
    y, A, B = orc.ffn_forward(x, W1, W3, W2, eti, off, tim, gates, act)
    dx, dW1, dW3, dW2 = orc.ffn_backward(dy, x, W1, W3, W2, eti, off, tim, gates, act)
    dz = orc.router_backward(dy, x, W1, W3, W2, eti, off, tei, tim, gates, act)
    return dict(tei=tei, gates=gates, eti=eti, off=off, tim=tim, y=y, A=A, B=B,
                dx=dx, dW1=dW1, dW3=dW3, dW2=dW2, dlogits=dz)


DENSE_CASES = [
    # L, d, h, E, K, act, int_logits   (d == h in some cases so that a
    # transposed weight would still run and has to be caught by value)
    (37, 6, 6, 5, 2, SWIGLU, False),
    (29, 5, 5, 4, 3, SILU, True),
    (23, 4, 7, 3, 3, SWIGLU, False),
    (31, 8, 3, 6, 1, SILU, False),
    (16, 3, 3, 8, 4, SWIGLU, True),
]


def check_dense_mask(orc):
    for i, (L, d, h, E, K, act, ints) in enumerate(DENSE_CASES):
        logits, x, W1, W3, W2, dy = tiny_inputs(L, d, h, E, K, act, 20 + i, ints)
        o = _run_oracle(orc, logits, x, W1, W3, W2, dy, K, act)
        ref = dense_mask_torch(logits, x, W1, W3, W2, dy, K, act)
        sel = np.zeros((L, E), dtype=bool)
        np.put_along_axis(sel, o["tei"].astype(np.int64), True, axis=1)
        assert np.array_equal(sel, ref["mask"]), i
        for name in ("y", "dx", "dW1", "dW2", "dlogits") + (("dW3",) if act == SWIGLU else ()):
            err = relerr(o[name], ref[name])
            assert err < 1e-6, (i, name, err)


def check_textbook_mlp(orc):
    """E = K = 1: the layer is y = act(x W1 [, x W3]) W2 (gate = 1)."""
    for act in (SILU, SWIGLU):
        logits, x, W1, W3, W2, dy = tiny_inputs(17, 5, 9, 1, 1, act, 5)
        o = _run_oracle(orc, logits, x, W1, W3, W2, dy, 1, act)
        xt = torch.tensor(x)
        a = xt @ torch.tensor(W1[0])
        G = F.silu(a) * (xt @ torch.tensor(W3[0])) if act == SWIGLU else F.silu(a)
        y = (G @ torch.tensor(W2[0])).numpy()
        assert relerr(o["y"], y) < 1e-12
        assert relerr(o["A"], a.numpy()) < 1e-12


def check_finite_differences(orc):
    for i, (L, d, h, E, K, act, ints) in enumerate(DENSE_CASES[:3]):
        logits, x, W1, W3, W2, dy = tiny_inputs(L, d, h, E, K, act, 40 + i, ints)
        E = W1.shape[0]
        tei, gates = orc.route(logits, K)
        eti, off, tim = orc.build_indices(tei, E)

        def loss(x_, W1_, W3_, W2_):
            y, _, _ = orc.ffn_forward(x_, W1_, W3_, W2_, eti, off, tim, gates, act)
            return float((y * dy).sum())

        dx, dW1, dW3, dW2 = orc.ffn_backward(dy, x, W1, W3, W2, eti, off, tim, gates, act)
        rng = np.random.default_rng(99 + i)
        eps = 1e-5
        args = {"x": x, "W1": W1, "W3": W3, "W2": W2}
        grads = {"x": dx, "W1": dW1, "W3": dW3, "W2": dW2}
        for name in ("x", "W1", "W2") + (("W3",) if act == SWIGLU else ()):
            for _ in range(2):
                V = rng.standard_normal(args[name].shape)
                plus = dict(args); minus = dict(args)
                plus[name] = args[name] + eps * V
                minus[name] = args[name] - eps * V
                fd = (loss(plus["x"], plus["W1"], plus["W3"], plus["W2"])
                      - loss(minus["x"], minus["W1"], minus["W3"], minus["W2"])) / (2 * eps)
                an = float((grads[name] * V).sum())
                assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (i, name, fd, an)


def check_sampled_consistency(orc):
    for i, (L, d, h, E, K, act, ints) in enumerate(DENSE_CASES):
        logits, x, W1, W3, W2, dy = tiny_inputs(L, d, h, E, K, act, 60 + i, ints)
        o = _run_oracle(orc, logits, x, W1, W3, W2, dy, K, act)
        # a sample in which several tokens share a slot's expert, and every token
        toks = np.array([L - 1, 0, L // 2, 1, 2, 3, L // 3, 5, 7])
        for tt in (toks, np.arange(L)):
            y, dx = orc.token_rows(tt, dy, x, W1, W3, W2, o["tei"], o["tim"], o["gates"], act)
            assert relerr(y, o["y"][tt]) < 1e-12, i
            assert relerr(dx, o["dx"][tt]) < 1e-12, i
        for prow in (np.array([L * K - 1, 0, L * K // 3, 1, 2, L * K // 2]), np.arange(L * K)):
            A, B = orc.route_rows_forward(prow, x, W1, W3, o["eti"], o["off"], act)
            assert relerr(A, o["A"][prow]) < 1e-12, i
            if act == SWIGLU:
                assert relerr(B, o["B"][prow]) < 1e-12, i
        for e in range(E):
            cols = np.array([0, h - 1])
            c1, c3, r2 = orc.dw_columns(e, cols, dy, x, W1, W3, W2, o["eti"], o["off"],
                                        o["tim"], o["tei"], o["gates"], act)
            assert np.allclose(c1, o["dW1"][e][:, cols], rtol=1e-12, atol=1e-13), (i, e)
            assert np.allclose(r2, o["dW2"][e][cols, :], rtol=1e-12, atol=1e-13), (i, e)
            if act == SWIGLU:
                assert np.allclose(c3, o["dW3"][e][:, cols], rtol=1e-12, atol=1e-13), (i, e)


def _gates64(logits, tei):
    """Softmax over each token's selected logits, in float64."""
    z = np.take_along_axis(np.asarray(logits, dtype=np.float64), np.asarray(tei, dtype=np.int64), axis=1)
    w = np.exp(z - z.max(axis=1, keepdims=True))
    return w / w.sum(axis=1, keepdims=True)


def check_router_finite_differences(orc):
    """<y, dy> as a function of the logits, with the selection held (the
    direction is small enough not to change any token's top K)."""
    for i, (L, d, h, E, K, act, ints) in enumerate(DENSE_CASES[:3]):
        if ints:
            continue
        logits, x, W1, W3, W2, dy = tiny_inputs(L, d, h, E, K, act, 140 + i)
        tei, _ = orc.route(logits, K)
        eti, off, tim = orc.build_indices(tei, E)
        z0 = np.asarray(logits, dtype=np.float64)

        def loss(z):
            y, _, _ = orc.ffn_forward(x, W1, W3, W2, eti, off, tim, _gates64(z, tei), act)
            return float((y * dy).sum())

        dz = orc.router_backward(dy, x, W1, W3, W2, eti, off, tei, tim, _gates64(z0, tei), act)
        rng = np.random.default_rng(7 + i)
        eps = 1e-6
        for _ in range(3):
            V = rng.standard_normal(z0.shape)
            for zz in (z0 + eps * V, z0 - eps * V):
                t2, _ = orc.route(zz.astype(np.float32), K)
                assert np.array_equal(t2, tei), "direction changed the selection"
            fd = (loss(z0 + eps * V) - loss(z0 - eps * V)) / (2 * eps)
            an = float((dz * V).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (i, fd, an)


def check_router_special_cases(orc):
    # K = 1: every gate is exactly 1, so the logits get no gradient
    logits, x, W1, W3, W2, dy = tiny_inputs(21, 4, 6, 5, 1, SWIGLU, 31)
    o = _run_oracle(orc, logits, x, W1, W3, W2, dy, 1, SWIGLU)
    assert np.all(o["dlogits"] == 0)
    # unselected logits get exactly 0; each row of a softmax Jacobian sums to 0
    logits, x, W1, W3, W2, dy = tiny_inputs(25, 5, 4, 6, 3, SILU, 32)
    o = _run_oracle(orc, logits, x, W1, W3, W2, dy, 3, SILU)
    sel = np.zeros(logits.shape, dtype=bool)
    np.put_along_axis(sel, o["tei"].astype(np.int64), True, axis=1)
    assert np.all(o["dlogits"][~sel] == 0)
    g64 = _gates64(logits, o["tei"])
    dz = orc.router_backward(dy, x, W1, W3, W2, o["eti"], o["off"], o["tei"], o["tim"], g64, SILU)
    assert np.abs(dz.sum(axis=1)).max() <= 1e-12 * max(1.0, np.abs(dz).max())
    # sampled rows agree with the full gradient (a few tokens; every token)
    for toks in (np.array([24, 0, 12, 1, 2, 3, 4]), np.arange(25)):
        rows = orc.router_rows(toks, dy, x, W1, W3, W2, o["tei"], o["gates"], SILU, 6)
        assert relerr(rows, o["dlogits"][toks]) < 1e-12
    logits, x, W1, W3, W2, dy = tiny_inputs(19, 5, 6, 4, 2, SWIGLU, 33)
    o = _run_oracle(orc, logits, x, W1, W3, W2, dy, 2, SWIGLU)
    toks = np.array([18, 3, 0, 7, 8, 9])
    rows = orc.router_rows(toks, dy, x, W1, W3, W2, o["tei"], o["gates"], SWIGLU, 4)
    assert relerr(rows, o["dlogits"][toks]) < 1e-12


def check_empty_expert(orc):
    logits, x, W1, W3, W2, dy = tiny_inputs(20, 4, 4, 4, 2, SWIGLU, 77)
    logits[:, 2] = -1e4                    # expert 2 never chosen
    o = _run_oracle(orc, logits, x, W1, W3, W2, dy, 2, SWIGLU)
    assert o["off"][3] == o["off"][2]
    assert np.all(o["dW1"][2] == 0) and np.all(o["dW3"][2] == 0) and np.all(o["dW2"][2] == 0)


def check_checkpoint_size(orc):
    logits, x, W1, W3, W2, dy = tiny_inputs(13, 4, 6, 3, 2, SWIGLU, 8)
    o = _run_oracle(orc, logits, x, W1, W3, W2, dy, 2, SWIGLU)
    assert orc.checkpoint_bytes(13, 2, 6, SWIGLU, 8) == o["A"].nbytes + o["B"].nbytes
    assert orc.checkpoint_bytes(13, 2, 6, SILU, 8) == o["A"].nbytes


ALL_CHECKS = [
    check_golden_dispatch,
    check_bruteforce_indices,
    check_invariants,
    check_special_cases_indices,
    check_gates_closed_forms,
    check_dense_mask,
    check_textbook_mlp,
    check_finite_differences,
    check_router_finite_differences,
    check_router_special_cases,
    check_sampled_consistency,
    check_empty_expert,
    check_checkpoint_size,
]
