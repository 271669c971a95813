"""Plant plausible mistakes in a copy of the oracle; the pins must catch each.

Every mutant is a textual edit of ``oracle/linattn.py`` loaded as a separate
module (the real oracle is untouched).  A mutant is caught when at least one
``check_*`` in ``tests/oracle_pins.py`` raises.  This is how the pins are shown
to constrain every term, sign, index and operand of the oracle.
"""
import importlib.util
import os
import types

import pytest

from tests import oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "linattn.py")

MUTANTS = {
    "mask_excludes_diagonal": ("keep = np.arange(n_cols)[None, :] <= np.arange(n_rows)[:, None]",
                               "keep = np.arange(n_cols)[None, :] < np.arange(n_rows)[:, None]"),
    "mask_transposed": ("keep = np.arange(n_cols)[None, :] <= np.arange(n_rows)[:, None]",
                        "keep = np.arange(n_cols)[None, :] >= np.arange(n_rows)[:, None]"),
    "chunked_unmasked_intra": ("sc = tril(qc @ kc.T)", "sc = qc @ kc.T"),
    "chunked_no_inter": ("num = qc @ S + sc @ vc", "num = sc @ vc"),
    "chunked_no_intra": ("num = qc @ S + sc @ vc", "num = qc @ S"),
    "chunked_state_before_read": ("        sc = tril(qc @ kc.T)\n",
                                  "        S = S + kc.T @ vc\n        sc = tril(qc @ kc.T)\n"),
    "chunked_wrong_sign": ("num = qc @ S + sc @ vc", "num = qc @ S - sc @ vc"),
    "chunked_den_no_intra": ("den = qc @ z + sc.sum(axis=1)", "den = qc @ z"),
    "chunked_den_no_inter": ("den = qc @ z + sc.sum(axis=1)", "den = sc.sum(axis=1)"),
    "chunked_z_not_updated": ("        z = z + kc.sum(axis=0)\n", "\n"),
    "chunked_drops_ragged_tail": ("for s in range(0, L, C):", "for s in range(0, L - C + 1, C):"),
    "chunked_no_clamp": ("    if C <= 0:\n        C = 1\n    q, k, v, integer = _prep(q, k, v)",
                         "    q, k, v, integer = _prep(q, k, v)"),
    "chunked_transposed_state": ("S = S + kc.T @ vc", "S = S + vc.T @ kc"),
    "recurrent_read_before_update": ("        S = S + np.outer(k[t], v[t])\n        z = z + k[t]\n        num = q[t] @ S\n",
                                     "        num = q[t] @ S\n        S = S + np.outer(k[t], v[t])\n        z = z + k[t]\n"),
    "recurrent_outer_swapped": ("S = S + np.outer(k[t], v[t])", "S = S + np.outer(v[t], k[t])"),
    "step_no_z": ("z = np.asarray(z, dtype=np.float64) + k_t", "z = np.asarray(z, dtype=np.float64)"),
    "prefix_form_off_by_one": ("S_pref = np.cumsum(k[:, :, None] * v[:, None, :], axis=0)",
                               "S_pref = np.cumsum(k[:, :, None] * v[:, None, :], axis=0) - k[:, :, None] * v[:, None, :]"),
    "scan_inclusive": ("        P[n] = run\n        run = run + Sf[n]\n", "        run = run + Sf[n]\n        P[n] = run\n"),
    "chunk_states_boundary": ("s, e = n * C, min((n + 1) * C, L)\n        S[n]", "s, e = n * C, min((n + 1) * C + 1, L)\n        S[n]"),
    "elu1_no_plus_one": ("np.where(x >= 0, x + 1.0, np.exp(np.minimum(x, 0.0)))",
                         "np.where(x >= 0, x, np.exp(np.minimum(x, 0.0)))"),
    "elu1_negative_branch": ("np.where(x >= 0, x + 1.0, np.exp(np.minimum(x, 0.0)))",
                             "np.where(x >= 0, x + 1.0, np.exp(np.minimum(x, 0.0)) - 1.0)"),
    "favor_sign": ("np.exp(proj - half_sq)", "np.exp(proj + half_sq)"),
    "favor_no_sqrt_m": ("np.exp(proj - half_sq) / np.sqrt(m)", "np.exp(proj - half_sq) / m"),
    "favor_full_norm": ("half_sq = 0.5 * np.sum(x * x, axis=-1, keepdims=True)",
                        "half_sq = np.sum(x * x, axis=-1, keepdims=True)"),
    "noncausal_state_transposed": ("    S = k.T @ v\n", "    S = v.T @ k\n"),
    "noncausal_scores_transposed": ("    A = q @ k.T\n", "    A = (q @ k.T).T\n"),
    "final_state_no_z": ("_finish(kf.sum(axis=0), integer)", "_finish(kf.sum(axis=0) * 0, integer)"),
    "brute_force_exclusive": ("last = i if causal else L - 1", "last = i - 1 if causal else L - 1"),
}

CHECKS = [getattr(pins, n) for n in dir(pins) if n.startswith("check_")]


def _load_mutant(old: str, new: str) -> types.ModuleType:
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) >= 1, f"mutation target not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = SRC
    exec(compile(src, SRC, "exec"), mod.__dict__)
    return mod


def _caught(mod) -> str:
    for check in CHECKS:
        try:
            if check is pins.check_exhaustive_tiny:
                check(mod, L=2)
            else:
                check(mod)
        except Exception as e:  # a crash on a planted mistake also counts as caught
            return f"{check.__name__}: {type(e).__name__}"
    return ""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    mod = _load_mutant(old, new)
    assert _caught(mod), f"no pin catches mutant {name}"


def test_unmutated_copy_passes():
    spec = importlib.util.spec_from_file_location("oracle_copy", SRC)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert _caught(mod) == ""
