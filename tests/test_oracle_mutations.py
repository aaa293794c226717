"""Plant one mistake at a time in a copy of the oracle (on the CPU) and check
that at least one pin fails.  This shows the pins are sharp enough to catch a
dropped term, a wrong sign, a wrong index or a transposed operand."""

import importlib.util
import os
import types

import pytest

import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "moe_oracle.py")

MUTATIONS = [
    ("ties to the higher expert id",
     'order = np.argsort(-logits, axis=1, kind="stable")',
     'order = logits.shape[1] - 1 - np.argsort(-logits[:, ::-1], axis=1, kind="stable")'),
    ("gates normalised by the max",
     "gates = (w / w.sum(axis=1, keepdims=True))",
     "gates = (w / w.max(axis=1, keepdims=True))"),
    ("offsets shifted by one expert",
     "offsets[1:] = np.cumsum(counts)",
     "offsets[:-1] = np.cumsum(counts)"),
    ("token_index_map of the wrong token",
     "tim = pos[tei, np.arange(L)[:, None]]",
     "tim = pos[tei, np.arange(L)[::-1, None]]"),
    ("gate applied to the wrong slot",
     "y += gates[:, k:k + 1] * O[tim[:, k]]",
     "y += gates[:, K - 1 - k:K - k] * O[tim[:, k]]"),
    ("SiLU sign",
     "return a / (1.0 + np.exp(-a))",
     "return a / (1.0 + np.exp(a))"),
    ("SiLU derivative sign",
     "return s * (1.0 + a * (1.0 - s))",
     "return s * (1.0 - a * (1.0 - s))"),
    ("transposed W2 in backward",
     "dG = dO[lo:hi] @ W2[e].T",
     "dG = dO[lo:hi] @ W2[e]"),
    ("dB uses SiLU(B)",
     "dB = dG * _silu(Ae)\n",
     "dB = dG * _silu(Be)\n"),
    ("gate dropped in backward",
     "dO[tim[:, k]] = gates[:, k:k + 1] * dy",
     "dO[tim[:, k]] = dy"),
    ("dx sums the first slot K times",
     "dx += dXr[tim[:, k]]",
     "dx += dXr[tim[:, 0]]"),
    ("dW1 from dB",
     "dW1[e] = X.T @ dA\n            dW3[e] = X.T @ dB",
     "dW1[e] = X.T @ dB\n            dW3[e] = X.T @ dB"),
    ("W1 and W3 roles swapped in SwiGLU",
     "return _silu(Ae) if act == SILU else _silu(Ae) * Be",
     "return _silu(Ae) if act == SILU else _silu(Be) * Ae"),
    ("sampled y without gate",
     "y[sel] += g * (G @ w2)",
     "y[sel] += (G @ w2)"),
    ("sampled A rows of the first selected expert only",
     "for e in np.unique(e_of):\n        sel = np.flatnonzero(e_of == e)",
     "for e in np.unique(e_of)[:1]:\n        sel = np.flatnonzero(e_of >= e)"),
    ("sampled dx with the slot's gate of slot 0",
     "gk = np.asarray(gates, dtype=np.float64)[tokens, k]",
     "gk = np.asarray(gates, dtype=np.float64)[tokens, 0]"),
    ("sampled router rows: tokens of one expert take the first token's output",
     "            dg[sel, k] = (DY[sel] * O).sum(axis=1)",
     "            dg[sel, k] = (DY[sel] * O[:1]).sum(axis=1)"),
    ("sampled dW2 rows without gate",
     "dO = g[:, None] * np.asarray(dy[toks], dtype=np.float64)",
     "dO = np.asarray(dy[toks], dtype=np.float64)"),
    ("router gradient without the softmax mean term",
     "    return gates * (dgate - s)",
     "    return gates * dgate"),
    ("router gradient from the gated output",
     "        dgate[:, k] = (dy * O[tim[:, k]]).sum(axis=1)",
     "        dgate[:, k] = (dy * gates[:, k:k + 1] * O[tim[:, k]]).sum(axis=1)"),
    ("router gradient in slot order instead of expert columns",
     "    np.put_along_axis(dz, np.asarray(tei, dtype=np.int64), _softmax_backward(gates, dgate), axis=1)",
     "    dz[:, :K] = _softmax_backward(gates, dgate)"),
]


def _mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    mod = _mutant(old, new)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no pin caught: {name}"
