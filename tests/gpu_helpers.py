"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI,
pull inputs back to the host, run the oracle on them, compare."""

from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
from token_dispatch_expert_amd import workloads as W
from token_dispatch_expert_amd.layer import MoELayerBuffers

SILU, SWIGLU = W.SILU, W.SWIGLU


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return torch.device("cuda:0")


def tol_of(cfg):
    """Max-relative error bound: 1e-5 for float32, 2e-2 for bf16 (float32
    accumulation)."""
    return 1e-5 if cfg.dtype == W.F32 else 2e-2


def host(t):
    """Device tensor -> float64 numpy (bf16 values upcast exactly)."""
    if t is None:
        return None
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def maxrel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / den)


# Every comparison made by assert_close: (test, tensor, max-rel, bound).
# conftest.py writes them out at the end of the session when
# MOE_PARITY_MARGINS names a file.
MARGINS = []


def _current_test():
    return os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]


def assert_close(name, got, ref, tol):
    err = maxrel(got, ref)
    say(f"    {name}: max-rel {err:.3e} (tol {tol:g})")
    MARGINS.append({"test": _current_test(), "tensor": name, "max_rel": err, "tol": tol,
                    "elements": int(np.asarray(ref).size)})
    assert np.all(np.isfinite(np.asarray(got, dtype=np.float64))), f"{name}: non-finite values"
    assert err <= tol, f"{name}: max-rel {err:.3e} > {tol:g}"


def oracle_dispatch(logits_host, cfg):
    tei, gates = oracle.route(logits_host, cfg.K)
    eti, off, tim = oracle.build_indices(tei, cfg.E)
    return dict(tei=tei, gates=gates, eti=eti, off=off, tim=tim)


def check_dispatch(buf: MoELayerBuffers, ref: dict, gate_tol=1e-6):
    """Indices bit-exact, gates within gate_tol (absolute, gates are in [0, 1])."""
    got = dict(tei=buf.tei.cpu().numpy(), eti=buf.eti.cpu().numpy(),
               off=buf.offsets.cpu().numpy(), tim=buf.tim.cpu().numpy())
    for k in ("off", "tei", "eti", "tim"):
        if not np.array_equal(got[k], ref[k]):
            bad = np.argwhere(np.asarray(got[k]).reshape(-1) != np.asarray(ref[k]).reshape(-1))
            raise AssertionError(f"{k} differs at {bad.size} positions, first {bad[:5].ravel()}")
    g = buf.gates.cpu().numpy().astype(np.float64)
    err = float(np.abs(g - ref["gates"].astype(np.float64)).max())
    say(f"    indices bit-exact; gates max-abs {err:.2e}")
    assert err <= gate_tol


def full_inputs_host(inp):
    return {k: host(v) if k != "logits" else v.cpu().numpy() for k, v in inp.items()}


def run_full_parity(cfg, seed, device, inp=None, check_determinism=False, recompute_g=False):
    """Whole-tensor parity for shapes the oracle runs in seconds."""
    inp = inp or W.make_inputs(cfg, seed, device)
    buf = MoELayerBuffers(cfg, device, router_grad=True, recompute_g=recompute_g)
    h_in = full_inputs_host(inp)
    ref = oracle_dispatch(h_in["logits"], cfg)
    buf.build(inp["logits"])
    buf.forward(inp["x"], inp["W1"], inp["W3"], inp["W2"])
    torch.cuda.synchronize()
    check_dispatch(buf, ref)
    A_gpu, B_gpu, y_gpu = host(buf.A), host(buf.B), host(buf.y)
    buf.backward(inp["dy"], inp["x"], inp["W1"], inp["W3"], inp["W2"])
    torch.cuda.synchronize()
    tol = tol_of(cfg)
    y, A, B = oracle.ffn_forward(h_in["x"], h_in["W1"], h_in["W3"], h_in["W2"], ref["eti"],
                                 ref["off"], ref["tim"], ref["gates"], cfg.act)
    dx, dW1, dW3, dW2 = oracle.ffn_backward(h_in["dy"], h_in["x"], h_in["W1"], h_in["W3"],
                                            h_in["W2"], ref["eti"], ref["off"], ref["tim"],
                                            ref["gates"], cfg.act)
    assert_close("A", A_gpu, A, tol)
    if cfg.act == SWIGLU:
        assert_close("B", B_gpu, B, tol)
    assert_close("y", y_gpu, y, tol)
    assert_close("dx", host(buf.dx), dx, tol)
    dz = oracle.router_backward(h_in["dy"], h_in["x"], h_in["W1"], h_in["W3"], h_in["W2"],
                                ref["eti"], ref["off"], ref["tei"], ref["tim"], ref["gates"],
                                cfg.act)
    assert_close("dlogits", host(buf.dlogits), dz, tol)
    gW1, gW2 = host(buf.dW1), host(buf.dW2)
    gW3 = host(buf.dW3)
    for e in range(cfg.E):
        if ref["off"][e + 1] == ref["off"][e]:
            assert np.all(gW1[e] == 0) and np.all(gW2[e] == 0), f"expert {e} empty but dW != 0"
            if gW3 is not None:
                assert np.all(gW3[e] == 0)
            continue
        assert_close(f"dW1[{e}]", gW1[e], dW1[e], tol)
        assert_close(f"dW2[{e}]", gW2[e], dW2[e], tol)
        if cfg.act == SWIGLU:
            assert_close(f"dW3[{e}]", gW3[e], dW3[e], tol)
    return buf


def _rows(t, idx):
    return host(t[torch.as_tensor(idx, device=t.device, dtype=torch.long)])


def _dw_columns_for(n_e, d, h, rng, budget=4e11):
    """Columns of dW1/dW3 (rows of dW2) to compare for an expert with n_e
    routes: all of them when the oracle's products stay within `budget`
    multiply-adds, else one aligned block of 256 (a whole output tile of each
    weight-gradient product) plus the first, the last and 14 random ones."""
    if n_e * d * h <= budget:
        return np.arange(h)
    blk = int(rng.integers(0, (h + 255) // 256)) * 256
    cols = np.concatenate([np.arange(blk, min(blk + 256, h)), [0, h - 1],
                           rng.integers(0, h, 14)])
    return np.unique(cols)


def run_sampled_parity(cfg, seed, device, n_tokens=4096, recompute_g=False):
    """Parity at full size on outputs the oracle computes from a subset of
    rows: indices in full; y, dx, dlogits and the A/B rows of n_tokens
    seeded tokens (plus the first and the last); dW1/dW3/dW2 of the
    heaviest, the lightest non-empty and one random other expert (whole
    matrices where the oracle runs them in seconds, else a column subset
    covering whole tiles), and exact zeros for every empty expert."""
    say(f"  sampled parity {cfg.name} seed {seed}" + (" (G formed in [L, h] pieces)" if recompute_g else ""))
    inp = W.make_inputs(cfg, seed, device)
    buf = MoELayerBuffers(cfg, device, router_grad=True, recompute_g=recompute_g)
    logits = inp["logits"].cpu().numpy()
    ref = oracle_dispatch(logits, cfg)
    buf.build(inp["logits"])
    buf.forward(inp["x"], inp["W1"], inp["W3"], inp["W2"])
    torch.cuda.synchronize()
    check_dispatch(buf, ref)
    rng = np.random.default_rng(1000 + seed)
    toks = np.unique(np.concatenate([[0, cfg.L - 1],
                                     rng.choice(cfg.L, size=min(n_tokens, cfg.L), replace=False)]))
    prow = ref["tim"][toks].reshape(-1)
    A_s = _rows(buf.A, prow)
    B_s = _rows(buf.B, prow) if cfg.act == SWIGLU else None
    y_s = _rows(buf.y, toks)
    buf.backward(inp["dy"], inp["x"], inp["W1"], inp["W3"], inp["W2"])
    torch.cuda.synchronize()
    dx_s = _rows(buf.dx, toks)
    dz_s = _rows(buf.dlogits, toks)
    tol = tol_of(cfg)
    say(f"    {toks.size} tokens, {prow.size} routes sampled")

    W1h, W2h = host(inp["W1"]), host(inp["W2"])
    W3h = host(inp["W3"])
    # token-row evaluation on compacted inputs (tokens renumbered 0..n-1)
    xs, dys = _rows(inp["x"], toks), _rows(inp["dy"], toks)
    y_r, dx_r = oracle.token_rows(np.arange(toks.size), dys, xs, W1h, W3h, W2h,
                                  ref["tei"][toks], None, ref["gates"][toks], cfg.act)
    # A/B of those routes: route p reads row eti_c[p] of the compacted xs
    eti_c = np.full(cfg.R, -1, dtype=np.int64)
    eti_c[prow] = np.searchsorted(toks, ref["eti"][prow])
    off = ref["off"].astype(np.int64)
    A_r, B_r = oracle.route_rows_forward(prow, xs, W1h, W3h, eti_c, off, cfg.act)
    assert_close("A rows", A_s, A_r, tol)
    if cfg.act == SWIGLU:
        assert_close("B rows", B_s, B_r, tol)
    del A_s, B_s, A_r, B_r
    assert_close("y rows", y_s, y_r, tol)
    assert_close("dx rows", dx_s, dx_r, tol)
    dz_r = oracle.router_rows(np.arange(toks.size), dys, xs, W1h, W3h, W2h, ref["tei"][toks],
                              ref["gates"][toks], cfg.act, cfg.E)
    assert_close("dlogits rows", dz_s, dz_r, tol)

    counts = np.diff(off)
    nonempty = np.flatnonzero(counts > 0)
    heavy = int(nonempty[np.argmax(counts[nonempty])])
    light = int(nonempty[np.argmin(counts[nonempty])])
    others = [int(e) for e in nonempty if e not in (heavy, light)]
    experts = [heavy, light] + ([int(rng.choice(others))] if others else [])
    for e in experts:
        lo, hi = int(off[e]), int(off[e + 1])
        cols = _dw_columns_for(hi - lo, cfg.d, cfg.h, rng)
        what = "all" if cols.size == cfg.h else f"{cols.size} of {cfg.h}"
        say(f"    expert {e}: {hi - lo} routes, {what} columns")
        etoks = ref["eti"][lo:hi]
        xe, dye = _rows(inp["x"], etoks), _rows(inp["dy"], etoks)
        off_c = np.zeros(cfg.E + 1, dtype=np.int64)
        off_c[e + 1:] = hi - lo
        c1, c3, r2 = oracle.dw_columns(e, cols, dye, xe, W1h, W3h, W2h,
                                       np.arange(hi - lo), off_c, None, ref["tei"][etoks],
                                       ref["gates"][etoks], cfg.act)
        del xe, dye
        gcols = torch.as_tensor(cols, device=device, dtype=torch.long)
        tag = "" if cols.size == cfg.h else "[cols]"
        assert_close(f"dW1[{e}]{tag}", host(buf.dW1[e][:, gcols]), c1, tol)
        assert_close(f"dW2[{e}]{tag}", host(buf.dW2[e][gcols, :]), r2, tol)
        if cfg.act == SWIGLU:
            assert_close(f"dW3[{e}]{tag}", host(buf.dW3[e][:, gcols]), c3, tol)
    empty = np.flatnonzero(counts == 0)
    for e in empty:
        assert int(torch.count_nonzero(buf.dW1[e])) == 0
        assert int(torch.count_nonzero(buf.dW2[e])) == 0
        if cfg.act == SWIGLU:
            assert int(torch.count_nonzero(buf.dW3[e])) == 0
        say(f"    empty expert {e}: dW exactly zero")
    return buf
