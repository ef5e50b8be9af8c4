"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU) and check
that at least one pin fails.  This is what makes the pins worth trusting: a
dropped term, a wrong sign or index, a transposed operand or a wrong log base
in the oracle would not go unnoticed."""

import importlib.util
import os
import types

import pytest

from tests import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention.py")

# (name, original text, mutated text, occurrence index or None for all)
MUTANTS = [
    ("causal off by one", "r[None, :] <= p[:, None]", "r[None, :] < p[:, None]", None),
    ("causal ignores offsets", "p = q_pos0 + np.arange", "p = 0 * q_pos0 + np.arange", None),
    ("forward drops scale", "s = scale * (q[r0:r1] @ k.T)", "s = (q[r0:r1] @ k.T)", 0),
    ("backward drops scale in scores", "s = scale * (q[r0:r1] @ k.T)", "s = (q[r0:r1] @ k.T)", 1),
    ("log base 2", "m_safe + np.log(l)", "m_safe + np.log2(l)", None),
    ("LSE forgets the max", "lse = np.where(any_vis, m_safe + np.log(l), -np.inf)",
     "lse = np.where(any_vis, np.log(l), -np.inf)", None),
    ("P not normalised", "e / np.where(any_vis, l, 1.0)[:, None]", "e", None),
    ("output uses keys", "O[r0:r1] = P @ v", "O[r0:r1] = P @ k[:, :v.shape[1]]", None),
    ("transposed score operand", "s = scale * (q[r0:r1] @ k.T)", "s = scale * (k @ q[r0:r1].T).T[:, ::-1]", 0),
    ("merge weights ignore LSE", "coef = np.where(live, np.exp(l - np.where(live, lse, 0.0)), 0.0)",
     "coef = np.where(live, 1.0 / len(parts), 0.0)", None),
    ("merge LSE drops max", "lse = np.where(live, m_safe + np.log(np.where(live, tot, 1.0)), -np.inf)",
     "lse = np.where(live, np.log(np.where(live, tot, 1.0)), -np.inf)", None),
    ("tree drops odd element", "nxt.append(level[-1])", "pass", None),
    ("backward drops D", "dS = P * (dP - D[r0:r1, None])", "dS = P * dP", None),
    ("backward sign of D", "dS = P * (dP - D[r0:r1, None])", "dS = P * (D[r0:r1, None] - dP)", None),
    ("dQ without scale", "dq[r0:r1] = scale * (dS @ k)", "dq[r0:r1] = (dS @ k)", None),
    ("dK from dS not transposed", "dk += scale * (dS.T @ q[r0:r1])", "dk += scale * (P.T @ q[r0:r1])", None),
    ("dV uses dP", "dv += P.T @ do[r0:r1]", "dv += dS.T @ do[r0:r1]", None),
    ("backward ignores mask",
     "P = np.where(vis & live[:, None], np.exp(np.where(vis, s, -np.inf) - lse_safe[:, None]), 0.0)",
     "P = np.where(live[:, None], np.exp(s - lse_safe[:, None]), 0.0)", None),
    ("delta from dO only", "D = np.sum(do * o, axis=1)", "D = np.sum(do, axis=1)", None),
    ("GQA interleaved mapping", "return h // (H_q // H_kv)", "return h % H_kv", None),
    ("GQA backward overwrites dK", "dk[b, :, g] += bk", "dk[b, :, g] = bk", None),
    ("GQA backward overwrites dV", "dv[b, :, g] += bv", "dv[b, :, g] = bv", None),
    ("GQA backward interleaved mapping", "g = _kv_head(h, H_q, H_kv)", "g = h % H_kv", 1),
    ("decode ignores seqlens", "n = L if seqlens is None else int(seqlens[b])", "n = L", None),
]


def _load_mutant(orig, new, occ):
    with open(SRC) as f:
        text = f.read()
    assert orig in text, f"mutation anchor not found: {orig}"
    if occ is None:
        text = text.replace(orig, new)
    else:
        parts = text.split(orig)
        assert len(parts) > occ + 1, "occurrence out of range"
        text = orig.join(parts[: occ + 1]) + new + orig.join(parts[occ + 1:])
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text, "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,orig,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, orig, new, occ):
    mod = _load_mutant(orig, new, occ)
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            failures.append((pin.__name__, type(exc).__name__))
    assert failures, f"mutant '{name}' passed every pin"
