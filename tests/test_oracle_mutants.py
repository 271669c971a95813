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
    # the decayed recurrence
    "decay_weights_transposed": ("e = np.arange(n_rows)[:, None] - np.arange(n_cols)[None, :]",
                                 "e = np.arange(n_cols)[None, :] - np.arange(n_rows)[:, None]"),
    "decay_weights_off_by_one": ("float(gamma) ** np.maximum(e, 0), 0.0)", "float(gamma) ** np.maximum(e + 1, 0), 0.0)"),
    "decay_recurrence_decays_input": ("        S = gamma * S + np.outer(k[t], v[t])\n",
                                      "        S = gamma * (S + np.outer(k[t], v[t]))\n"),
    "decay_recurrence_z_not_decayed": ("        z = gamma * z + k[t]\n", "        z = z + k[t]\n"),
    "decay_step_no_decay": ("S = gamma * np.asarray(S, dtype=np.float64) + np.outer(k_t, v_t)",
                            "S = np.asarray(S, dtype=np.float64) + np.outer(k_t, v_t)"),
    "decay_step_z_not_decayed": ("z = gamma * np.asarray(z, dtype=np.float64) + k_t",
                                 "z = np.asarray(z, dtype=np.float64) + k_t"),
    "decay_chunked_inter_exponent": ("g_in = float(gamma) ** (rows + 1)", "g_in = float(gamma) ** rows"),
    "decay_chunked_out_weight": ("g_out = float(gamma) ** (n - 1 - rows)", "g_out = float(gamma) ** (n - rows)"),
    "decay_chunked_carry_full_chunk": ("S = float(gamma) ** n * S + kc.T @ (g_out[:, None] * vc)",
                                       "S = float(gamma) ** C * S + kc.T @ (g_out[:, None] * vc)"),
    "decay_chunked_z_carry": ("z = float(gamma) ** n * z + (g_out[:, None] * kc).sum(axis=0)",
                              "z = z + (g_out[:, None] * kc).sum(axis=0)"),
    "decay_chunked_den_no_decay": ("den = g_in * (qc @ z) + sc.sum(axis=1)", "den = (qc @ z) + sc.sum(axis=1)"),
    "decay_chunk_states_weight": ("w = float(gamma) ** (e - 1 - np.arange(s, e))", "w = float(gamma) ** (e - np.arange(s, e))"),
    "decay_scan_length_index": ("run = float(gamma) ** int(lengths[n]) * run + Sf[n]",
                                "run = float(gamma) ** int(lengths[n - 1]) * run + Sf[n]"),
    "decay_scan_inclusive": ("        P[n] = run\n        run = float(gamma)",
                             "        P[n] = float(gamma) ** int(lengths[n]) * run + Sf[n]\n        run = float(gamma)"),
    "brute_force_decay_exponent": ("acc += g ** (i - j) * s * exact(v[j][c])", "acc += g ** (i - j + 1) * s * exact(v[j][c])"),
    "softmax_no_normalisation": ("    w = w / w.sum(axis=1, keepdims=True)\n", "\n"),
    "softmax_no_scale": ("    s = (q @ k.T) * scale\n", "    s = q @ k.T\n"),
    "softmax_causal_exclusive": ("keep = np.arange(k.shape[0])[None, :] <= np.arange(q.shape[0])[:, None]\n        s = np.where",
                                 "keep = np.arange(k.shape[0])[None, :] < np.arange(q.shape[0])[:, None]\n        s = np.where"),
    "loglinear_level_off_by_one": ("return 0 if s == t else int(t ^ s).bit_length()",
                                   "return 0 if s == t else int(t ^ s).bit_length() - 1"),
    "loglinear_merge_skips_level0": ("            merged = S[:b + 1].sum(axis=0)\n",
                                     "            merged = S[1:b + 1].sum(axis=0)\n"),
    "loglinear_merge_one_level_low": ("            S[b + 1] = merged\n", "            S[b] = merged\n"),
    "loglinear_resume_ignores_start": ("        t = t0 + i\n", "        t = i\n"),
    "loglinear_state_keeps_merged_levels": ("            S[1:b + 1] = 0.0\n", "\n"),
    "loglinear_bucket_shifted": ("Sb = sum(states[c_] for c_ in range(h - (1 << (m - 1)), h))",
                                 "Sb = sum(states[c_] for c_ in range(h - (1 << (m - 1)), h + 1) if c_ < n)"),
    "loglinear_chunk_level_index": ("acc = acc + lam[s:e, cb + m][:, None] * (q[s:e] @ Sb)",
                                    "acc = acc + lam[s:e, cb + m - 1][:, None] * (q[s:e] @ Sb)"),
    "loglinear_masked_wrong_level": ("            M[t, s_] = lam[t, loglinear_level(t, s_)]",
                                     "            M[t, s_] = lam[s_, loglinear_level(t, s_)]"),
    "apply_phi_drops_in_scale": ("        x = np.asarray(x, dtype=np.float64) * in_scale\n",
                                 "        x = np.asarray(x, dtype=np.float64)\n"),
    "apply_phi_scale_after_map": ("    if in_scale != 1.0:\n        x = np.asarray(x, dtype=np.float64) * in_scale\n"
                                  "    if fmap == \"identity\":\n        return phi_identity(x)\n"
                                  "    if fmap == \"elu1\":\n        return phi_elu1(x)\n",
                                  "    if fmap == \"identity\":\n        return phi_identity(x) * in_scale\n"
                                  "    if fmap == \"elu1\":\n        return phi_elu1(x) * in_scale\n"),
    "apply_phi_favor_scale_after_map": ("        return phi_favor(x, W)\n",
                                        "        return phi_favor(x / in_scale, W) * in_scale\n"),
    "forward_skips_scaled_identity": ("if (fmap != \"identity\" or in_scale != 1.0) else q_raw",
                                      "if fmap != \"identity\" else q_raw"),
    "forward_noncausal_ignores_normalize": ("    out = noncausal_state_first(qp, kp, v, normalize)\n",
                                            "    out = noncausal_state_first(qp, kp, v, False)\n"),
    "forward_noncausal_is_causal": ("    out = noncausal_state_first(qp, kp, v, normalize)\n",
                                    "    out = chunked(qp, kp, v, C, normalize)[0]\n"),
    "forward_noncausal_state_transposed": ("    S, z = final_state(kp, v)\n", "    S, z = final_state(v, kp)\n"),
    # the delta rule
    "delta_read_before_update": ("        S = old + np.outer(k[t], u)          # erase along k_t and write\n        out[t] = q[t] @ S\n",
                                 "        out[t] = q[t] @ old\n        S = old + np.outer(k[t], u)\n"),
    "delta_no_erase": ("        u = b[t] * (v[t] - k[t] @ old)       # the new value minus the old prediction at k_t\n",
                       "        u = b[t] * v[t]\n"),
    "delta_erase_undecayed_state": ("        u = b[t] * (v[t] - k[t] @ old)       # the new value minus the old prediction at k_t\n",
                                    "        u = b[t] * (v[t] - k[t] @ S)\n"),
    "delta_beta_on_write_only": ("        u = b[t] * (v[t] - k[t] @ old)       # the new value minus the old prediction at k_t\n",
                                 "        u = b[t] * v[t] - k[t] @ old\n"),
    "delta_gate_on_write": ("        S = old + np.outer(k[t], u)          # erase along k_t and write\n",
                            "        S = a[t] * (S + np.outer(k[t], u))\n"),
    "delta_step_no_gate": ("    old = float(alpha_t) * np.asarray(S, dtype=np.float64)\n",
                           "    old = np.asarray(S, dtype=np.float64)\n"),
    "delta_step_read_before": ("    return np.asarray(q_t, dtype=np.float64) @ S, S\n",
                               "    return np.asarray(q_t, dtype=np.float64) @ old, S\n"),
    "delta_solve_sign": ("        X[i] = R[i] - A[i, :i] @ X[:i]\n", "        X[i] = R[i] + A[i, :i] @ X[:i]\n"),
    "delta_chunked_A_upper": ("        A = np.tril(bc[:, None] * (kc @ kc.T) * G, -1)\n",
                              "        A = np.triu(bc[:, None] * (kc @ kc.T) * G, 1).T\n"),
    "delta_chunked_A_beta_on_columns": ("        A = np.tril(bc[:, None] * (kc @ kc.T) * G, -1)\n",
                                        "        A = np.tril(bc[None, :] * (kc @ kc.T) * G, -1)\n"),
    "delta_chunked_G_transposed": ("        G = g[:, None] / g[None, :]\n", "        G = g[None, :] / g[:, None]\n"),
    "delta_chunked_no_gate_on_inter": ("        out[s:e] = g[:, None] * (qc @ P) + (tril(qc @ kc.T) * G) @ U\n",
                                       "        out[s:e] = (qc @ P) + (tril(qc @ kc.T) * G) @ U\n"),
    "delta_chunked_intra_exclusive": ("        out[s:e] = g[:, None] * (qc @ P) + (tril(qc @ kc.T) * G) @ U\n",
                                      "        out[s:e] = g[:, None] * (qc @ P) + (np.tril(qc @ kc.T, -1) * G) @ U\n"),
    "delta_chunked_carry_undecayed": ("        P = g[-1] * P + kc.T @ ((g[-1] / g)[:, None] * U)\n",
                                      "        P = P + kc.T @ ((g[-1] / g)[:, None] * U)\n"),
    "delta_chunked_carry_weights": ("        P = g[-1] * P + kc.T @ ((g[-1] / g)[:, None] * U)\n",
                                    "        P = g[-1] * P + kc.T @ U\n"),
    "delta_chunked_rhs_ungated": ("        U = unit_lower_solve(A, bc[:, None] * (vc - g[:, None] * (kc @ P)))\n",
                                  "        U = unit_lower_solve(A, bc[:, None] * (vc - (kc @ P)))\n"),
    "delta_transform_no_beta": ("        out.append(unit_lower_solve(A, np.diag(b[s:e])))\n",
                                "        out.append(unit_lower_solve(A, np.eye(e - s)))\n"),
    "delta_transform_ungated": ("        A = np.tril(b[s:e, None] * (k[s:e] @ k[s:e].T) * (g[:, None] / g[None, :]), -1)\n",
                                "        A = np.tril(b[s:e, None] * (k[s:e] @ k[s:e].T), -1)\n"),
    "brute_force_delta_ungated": ("        S = [[at * S[i][c] for c in range(dv)] for i in range(dk)]\n",
                                  "        S = [[S[i][c] for c in range(dv)] for i in range(dk)]\n"),
    "brute_force_delta_no_erase": ("        u = [bt * (exact(v[t][c]) - pred[c]) for c in range(dv)]\n",
                                   "        u = [bt * exact(v[t][c]) for c in range(dv)]\n"),
    "forward_ignores_gamma": ("        return decay_chunked(qp, kp, v, C, gamma, normalize)",
                              "        return chunked(qp, kp, v, C, normalize)"),
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
