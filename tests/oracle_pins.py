"""Checks that pin the CPU oracle to what the pages and the mathematics fix.

Each ``check_*`` takes the oracle module and raises AssertionError on a
violation.  ``tests/test_oracle_pins.py`` runs them on the real oracle;
``tests/test_oracle_mutants.py`` plants plausible mistakes in a copy of the
oracle and requires that at least one check fails for every mistake.

Pages: the chunking page is "attention と線形の間"
(sharin-2a1.pages.dev/parts/chunked.html); the linear-attention page is
"Linear Attention / Performerの理論と実装" (disassemble-channel.com/linear-attention/).
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np

from workloads import bf16_bits_to_f64, f32_to_bf16_bits


def _ints(rng, shape, lo=-3, hi=3):
    return rng.integers(lo, hi + 1, size=shape).astype(np.int64)


def _bf16(rng, shape, scale=1.0):
    return bf16_bits_to_f64(f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * scale))


def _frac_matrix(m):
    return np.array([[float(x) for x in row] for row in m])


# ---------------------------------------------------------------------------
# P-a / P-c: the forms agree exactly on integers, for every chunk size
# ---------------------------------------------------------------------------
def check_exhaustive_tiny(o, L: int = 2, vals=(-1, 0, 1)) -> None:
    """All q, k, v in {-1,0,1}^(L x 1): scores-first, state-first, the materialised
    prefix form, chunked for every C in 0..L+1 and brute force agree exactly
    (chunking page, section ②: both ends and every chunk size give one answer)."""
    for flat in itertools.product(vals, repeat=3 * L):
        a = np.array(flat, dtype=np.int64).reshape(3, L, 1)
        q, k, v = a[0], a[1], a[2]
        ref = o.causal_scores_first(q, k, v)
        bf = np.array([[int(x) for x in row] for row in o.brute_force(q, k, v)], dtype=np.int64)
        assert np.array_equal(ref, bf), (flat, ref, bf)
        rec, S, z = o.causal_state_first(q, k, v)
        assert np.array_equal(rec, ref), flat
        assert np.array_equal(o.causal_materialized_prefix(q, k, v), ref), flat
        for C in range(0, L + 2):
            ch, Sc, zc = o.chunked(q, k, v, C)
            assert np.array_equal(ch, ref), (flat, C)
            assert np.array_equal(Sc, S) and np.array_equal(zc, z), (flat, C)


def check_random_int_all_chunks(o, seed: int = 0) -> None:
    """Random integers, d_k != d_v, every C from 0 to L+3 including non-divisors."""
    rng = np.random.default_rng([seed, 11])
    L, dk, dv = 23, 5, 3
    q, k, v = _ints(rng, (L, dk)), _ints(rng, (L, dk)), _ints(rng, (L, dv))
    ref = o.causal_scores_first(q, k, v)
    bf = np.array([[int(x) for x in row] for row in o.brute_force(q, k, v)], dtype=np.int64)
    assert np.array_equal(ref, bf)
    rec, S, z = o.causal_state_first(q, k, v)
    assert np.array_equal(rec, ref)
    # final state: S = sum_t k_t^T v_t (d_k x d_v), z = sum_t k_t
    S_def = sum(np.outer(k[t], v[t]) for t in range(L))
    assert S.shape == (dk, dv) and np.array_equal(S, S_def)
    assert np.array_equal(z, k.sum(axis=0))
    Sf, zf = o.final_state(k, v)
    assert np.array_equal(Sf, S_def) and np.array_equal(zf, z)
    for C in range(0, L + 4):
        ch, Sc, zc = o.chunked(q, k, v, C)
        assert np.array_equal(ch, ref), C
        assert np.array_equal(Sc, S_def) and np.array_equal(zc, z), C


def check_chunk_phases(o, seed: int = 1) -> None:
    """Per-chunk states are k_c^T v_c of each chunk; the exclusive prefix P_n sums
    the chunks before n; the total is the final state; out_c = q_c P_n + tril(q_c k_c^T) v_c."""
    rng = np.random.default_rng([seed, 12])
    L, dk, dv = 29, 4, 6
    q, k, v = _ints(rng, (L, dk)), _ints(rng, (L, dk)), _ints(rng, (L, dv))
    for C in (1, 4, 7, 29, 40):
        Sn, zn = o.chunk_states(k, v, C)
        N = (L + C - 1) // C
        assert Sn.shape == (N, dk, dv) and zn.shape == (N, dk)
        for n in range(N):
            rows = range(n * C, min((n + 1) * C, L))
            assert np.array_equal(Sn[n], sum(np.outer(k[t], v[t]) for t in rows))
            assert np.array_equal(zn[n], sum(k[t] for t in rows))
        P, total = o.exclusive_scan(Sn)
        assert np.array_equal(P[0], np.zeros((dk, dv)))
        for n in range(1, N):
            assert np.array_equal(P[n], Sn[:n].sum(axis=0))
        assert np.array_equal(total, o.final_state(k, v)[0])
        ref = o.causal_scores_first(q, k, v)
        for n in range(N):
            s, e = n * C, min((n + 1) * C, L)
            blk = q[s:e] @ P[n] + o.tril(q[s:e] @ k[s:e].T) @ v[s:e]
            assert np.array_equal(blk, ref[s:e]), (C, n)


def check_brute_force_float(o, seed: int = 2) -> None:
    """bf16-valued floats: the float64 forms match exact rational arithmetic to
    float64 rounding, normalised and not."""
    rng = np.random.default_rng([seed, 13])
    L, dk, dv = 9, 3, 2
    q, k, v = _bf16(rng, (L, dk)), _bf16(rng, (L, dk)), _bf16(rng, (L, dv))
    qp, kp = o.phi_elu1(q), o.phi_elu1(k)
    for normalize in (False, True):
        exact = _frac_matrix(o.brute_force(qp, kp, v, causal=True, normalize=normalize))
        forms = [o.causal_scores_first(qp, kp, v, normalize),
                 o.causal_state_first(qp, kp, v, normalize)[0],
                 o.causal_materialized_prefix(qp, kp, v, normalize)]
        forms += [o.chunked(qp, kp, v, C, normalize)[0] for C in (1, 2, 4, 9)]
        for f in forms:
            assert np.allclose(f, exact, rtol=1e-12, atol=1e-12), (normalize, f, exact)
        exact_nc = _frac_matrix(o.brute_force(qp, kp, v, causal=False, normalize=normalize))
        assert np.allclose(o.noncausal_state_first(qp, kp, v, normalize), exact_nc, rtol=1e-12, atol=1e-12)
        assert np.allclose(o.noncausal_scores_first(qp, kp, v, normalize), exact_nc, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# P-b: the two association orders (chunking page, section ①)
# ---------------------------------------------------------------------------
def check_association_orders(o, seed: int = 3) -> None:
    rng = np.random.default_rng([seed, 14])
    for L, dk, dv in ((4, 2, 2), (17, 6, 3), (40, 8, 8)):
        q, k, v = _ints(rng, (L, dk)), _ints(rng, (L, dk)), _ints(rng, (L, dv))
        a = o.noncausal_scores_first(q, k, v)
        b = o.noncausal_state_first(q, k, v)
        assert np.array_equal(a, b)
        direct = np.array([[sum(int(q[i] @ k[j]) * int(v[j, c]) for j in range(L)) for c in range(dv)]
                           for i in range(L)])
        assert np.array_equal(a, direct)


# ---------------------------------------------------------------------------
# P-g, P-h, P-i, P-j: structural invariants
# ---------------------------------------------------------------------------
def check_last_row(o, seed: int = 4) -> None:
    """The last causal row sees every token, so it equals the last non-causal row
    (the page's printed pair shares its last row, [18 20])."""
    rng = np.random.default_rng([seed, 15])
    q, k, v = _ints(rng, (12, 3)), _ints(rng, (12, 3)), _ints(rng, (12, 4))
    assert np.array_equal(o.causal_scores_first(q, k, v)[-1], o.noncausal_state_first(q, k, v)[-1])
    qf, kf, vf = (_bf16(rng, (12, 3)), _bf16(rng, (12, 3)), _bf16(rng, (12, 4)))
    qf, kf = o.phi_elu1(qf), o.phi_elu1(kf)
    a = o.chunked(qf, kf, vf, 5, True)[0][-1]
    b = o.noncausal_state_first(qf, kf, vf, True)[-1]
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def check_causality(o, seed: int = 5) -> None:
    """Changing token t's q, k or v changes no output row before t."""
    rng = np.random.default_rng([seed, 16])
    L, dk, dv = 15, 3, 3
    q, k, v = _ints(rng, (L, dk)), _ints(rng, (L, dk)), _ints(rng, (L, dv))
    base = o.chunked(q, k, v, 4)[0]
    for t in (0, 3, 4, 9, 14):
        for which in range(3):
            arrs = [q.copy(), k.copy(), v.copy()]
            arrs[which][t] += 5
            pert = o.chunked(*arrs, 4)[0]
            assert np.array_equal(pert[:t], base[:t]), (t, which)
    # and the diagonal is included: changing v_t changes row t when q_t . k_t != 0
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[6] = k2[6] = np.array([1, 0, 0])
    v3 = v2.copy()
    v3[6] += 1
    assert not np.array_equal(o.chunked(q2, k2, v2, 4)[0][6], o.chunked(q2, k2, v3, 4)[0][6])


def check_linearity_and_normalised_cases(o, seed: int = 6) -> None:
    """Unnormalised output is linear in v (exactly, on integers).  Normalised
    output with positive features: o_0 = v_0, and each o_i lies coordinate-wise
    within [min_{j<=i} v_j, max_{j<=i} v_j] (a convex combination of past values)."""
    rng = np.random.default_rng([seed, 17])
    L, dk, dv = 14, 3, 4
    q, k = _ints(rng, (L, dk)), _ints(rng, (L, dk))
    v1, v2 = _ints(rng, (L, dv)), _ints(rng, (L, dv))
    for C in (1, 3, 14):
        f = lambda vv: o.chunked(q, k, vv, C)[0]
        assert np.array_equal(f(v1 + 2 * v2), f(v1) + 2 * f(v2))
    qf, kf, vf = o.phi_elu1(_bf16(rng, (L, dk))), o.phi_elu1(_bf16(rng, (L, dk))), _bf16(rng, (L, dv))
    for C in (1, 5, 14):
        out = o.chunked(qf, kf, vf, C, True)[0]
        assert np.allclose(out[0], vf[0], rtol=1e-14, atol=0)
        for i in range(L):
            lo, hi = vf[: i + 1].min(axis=0), vf[: i + 1].max(axis=0)
            assert np.all(out[i] >= lo - 1e-12) and np.all(out[i] <= hi + 1e-12)


def check_query_scale_invariance(o, seed: int = 7) -> None:
    """Normalised output does not change when each phi(q_i) is multiplied by a
    positive factor (so FAVOR+'s exp(-|q|^2/2)/sqrt(m) factor cancels)."""
    rng = np.random.default_rng([seed, 18])
    L, dk, dv = 11, 4, 3
    qf, kf, vf = o.phi_elu1(_bf16(rng, (L, dk))), o.phi_elu1(_bf16(rng, (L, dk))), _bf16(rng, (L, dv))
    s = np.exp(rng.standard_normal((L, 1)))
    for C in (1, 4, 11):
        a = o.chunked(qf, kf, vf, C, True)[0]
        b = o.chunked(qf * s, kf, vf, C, True)[0]
        assert np.allclose(a, b, rtol=1e-12, atol=1e-14)
        # the unnormalised output does scale
        a0 = o.chunked(qf, kf, vf, C, False)[0]
        b0 = o.chunked(qf * s, kf, vf, C, False)[0]
        assert np.allclose(b0, a0 * s, rtol=1e-12, atol=1e-14)


def check_recurrent_vs_prefix_page_inputs(o) -> None:
    """The linear-attention page checks its recurrent form against its
    materialised-prefix form on inputs from numpy's legacy generator, seed 42,
    n = 32, d_k = d_v = 16, scaled by 0.5, with elu+1 features and the
    normaliser, and reports agreement to floating-point error."""
    rs = np.random.RandomState(42)
    Q = rs.randn(32, 16) * 0.5
    K = rs.randn(32, 16) * 0.5
    V = rs.randn(32, 16) * 0.5
    qp, kp = o.phi_elu1(Q), o.phi_elu1(K)
    rec = o.causal_state_first(qp, kp, V, True)[0]
    par = o.causal_materialized_prefix(qp, kp, V, True)
    assert np.max(np.abs(rec - par)) < 1e-12
    quad = o.causal_scores_first(qp, kp, V, True)
    assert np.max(np.abs(rec - quad)) < 1e-12


def check_resume(o, seed: int = 8) -> None:
    """Forward over the first L1 tokens, then token-by-token steps from its final
    state, equals the forward over all L tokens (exact on integers)."""
    rng = np.random.default_rng([seed, 19])
    L, L1, dk, dv = 20, 13, 3, 5
    q, k, v = _ints(rng, (L, dk)), _ints(rng, (L, dk)), _ints(rng, (L, dv))
    full = o.chunked(q, k, v, 4)[0]
    _, S, z = o.chunked(q[:L1], k[:L1], v[:L1], 4)
    tail, _, _ = o.causal_state_first(q[L1:], k[L1:], v[L1:], False, S0=S, z0=z)
    assert np.array_equal(tail, full[L1:])
    # normalised decode steps on floats
    qf, kf, vf = o.phi_elu1(_bf16(rng, (L, dk))), o.phi_elu1(_bf16(rng, (L, dk))), _bf16(rng, (L, dv))
    fullf = o.chunked(qf, kf, vf, 6, True)[0]
    _, S, z = o.chunked(qf[:L1], kf[:L1], vf[:L1], 6, True)
    for t in range(L1, L):
        ot, S, z = o.recurrent_step(S, z, qf[t], kf[t], vf[t], True)
        assert np.allclose(ot, fullf[t], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# P-l: feature maps against closed forms
# ---------------------------------------------------------------------------
def check_elu1(o) -> None:
    x = np.array([-3.0, -1.0, -0.5, 0.0, 0.25, 1.0, 2.0])
    want = np.array([math.exp(-3.0), math.exp(-1.0), math.exp(-0.5), 1.0, 1.25, 2.0, 3.0])
    assert np.allclose(o.phi_elu1(x), want, rtol=1e-15, atol=0)
    big = np.linspace(-20, 20, 4001)
    assert np.all(o.phi_elu1(big) > 0)


def check_favor_closed_form(o) -> None:
    """phi(x)_l = exp(w_l.x - |x|^2/2)/sqrt(m), checked at hand-computed points."""
    d, m = 3, 4
    W = np.array([[1.0, 0, 0], [0, 1.0, 0], [0, 0, 1.0], [1.0, -1.0, 2.0]])
    x0 = np.zeros(d)
    assert np.allclose(o.phi_favor(x0, W), np.full(m, 0.5), rtol=1e-15)
    x = np.array([1.0, 2.0, -1.0])  # |x|^2 / 2 = 3
    want = np.array([math.exp(1 - 3), math.exp(2 - 3), math.exp(-1 - 3), math.exp((1 - 2 - 2) - 3)]) / 2.0
    assert np.allclose(o.phi_favor(x, W), want, rtol=1e-15)
    xs = np.stack([x0, x])
    assert np.allclose(o.phi_favor(xs, W)[1], want, rtol=1e-15)


def check_favor_convergence(o) -> None:
    """phi(q).phi(k) is an unbiased estimate of exp(q.k) for Gaussian rows; with
    many rows it converges (the page's moment-generating-function argument)."""
    from workloads import orthogonal_random_features
    q = np.array([0.3, -0.2, 0.1, 0.4])
    k = np.array([-0.1, 0.5, 0.2, 0.3])
    target = math.exp(float(q @ k))
    rng = np.random.default_rng([9, 20])
    W = rng.standard_normal((400000, 4))
    est = float(o.phi_favor(q, W) @ o.phi_favor(k, W))
    assert abs(est / target - 1) < 0.01, (est, target)
    _, Wo = orthogonal_random_features(65536, 4, [9, 21])
    est_o = float(o.phi_favor(q, Wo) @ o.phi_favor(k, Wo))
    assert abs(est_o / target - 1) < 0.02, (est_o, target)
    assert np.all(o.phi_favor(rng.standard_normal((10, 4)), W[:64]) > 0)


# ---------------------------------------------------------------------------
# Retention decay (linear-attention page, RNN view: S_t = gamma S_{t-1} +
# phi(k_t) v_t^T).  The recurrence is the definition; every other form is
# pinned to it, to exact brute force and to closed forms.  gamma = 1/2 and 3/4
# keep every weight a short binary fraction, so on small integers the float64
# forms are exact and must agree bit for bit.
# ---------------------------------------------------------------------------
def check_decay_reduces_to_plain(o, seed: int = 30) -> None:
    """gamma = 1 gives back plain linear attention in every form (exact on ints)."""
    rng = np.random.default_rng([seed, 31])
    L, dk, dv = 17, 3, 4
    q, k, v = _ints(rng, (L, dk)), _ints(rng, (L, dk)), _ints(rng, (L, dv))
    ref, S, z = o.causal_state_first(q, k, v)
    out, Sd, zd = o.decay_state_first(q, k, v, 1.0)
    assert np.array_equal(out, ref) and np.array_equal(Sd, S) and np.array_equal(zd, z)
    assert np.array_equal(o.decay_scores_first(q, k, v, 1.0), ref)
    for C in (1, 3, 5, 17, 20):
        out, Sd, zd = o.decay_chunked(q, k, v, C, 1.0)
        assert np.array_equal(out, ref) and np.array_equal(Sd, S) and np.array_equal(zd, z), C
        Sn, zn, lens = o.decay_chunk_states(k, v, C, 1.0)
        Sp, zp = o.chunk_states(k, v, C)
        assert np.array_equal(Sn, Sp) and np.array_equal(zn, zp), C
        P, tot = o.decay_exclusive_scan(Sn, lens, 1.0)
        Pp, totp = o.exclusive_scan(Sp)
        assert np.array_equal(P, Pp) and np.array_equal(tot, totp), C


def check_decay_forms_exact(o, seed: int = 32) -> None:
    """Dyadic gamma on small integers: the recurrence, the unrolled matrix form,
    the chunked form at every C (0..L+1, non-divisors included) and exact
    brute force agree exactly, normalised or not; the final states agree too."""
    rng = np.random.default_rng([seed, 33])
    L, dk, dv = 11, 2, 3
    for gamma in (Fraction(1, 2), Fraction(3, 4)):
        g = float(gamma)
        q, k, v = _ints(rng, (L, dk)), _ints(rng, (L, dk)), _ints(rng, (L, dv))
        ref, S, z = o.decay_state_first(q, k, v, g)
        bf = _frac_matrix(o.brute_force_decay(q, k, v, gamma))
        assert np.array_equal(ref, bf), gamma
        assert np.array_equal(o.decay_scores_first(q, k, v, g), ref), gamma
        for C in range(0, L + 2):
            out, Sc, zc = o.decay_chunked(q, k, v, C, g)
            assert np.array_equal(out, ref), (gamma, C)
            assert np.array_equal(Sc, S) and np.array_equal(zc, z), (gamma, C)
        # normalised, positive keys and queries (denominators away from zero)
        qp, kp = np.abs(q) + 1, np.abs(k) + 1
        refn = o.decay_state_first(qp, kp, v, g, True)[0]
        bfn = _frac_matrix(o.brute_force_decay(qp, kp, v, gamma, True))
        assert np.allclose(refn, bfn, rtol=1e-14, atol=0), gamma
        assert np.allclose(o.decay_scores_first(qp, kp, v, g, True), refn, rtol=1e-14, atol=0)
        for C in (1, 4, 7, L):
            assert np.allclose(o.decay_chunked(qp, kp, v, C, g, True)[0], refn, rtol=1e-14, atol=0), (gamma, C)


def check_decay_closed_forms(o) -> None:
    """d = 1, q = k = v = 1: y_t = sum_{j<=t} gamma^(t-j) = (1 - gamma^(t+1)) / (1 - gamma)
    (a geometric series), the final state is the same sum at t = L-1, the
    normalised output is 1; and y_t changes by gamma^t (q_t . k_0) delta when
    v_0 does (older tokens fade by one factor per step)."""
    L, gamma = 40, 0.9
    ones = np.ones((L, 1))
    t = np.arange(L)
    geo = (1 - gamma ** (t + 1)) / (1 - gamma)
    for C in (1, 7, 16, L):
        out, S, z = o.decay_chunked(ones, ones, ones, C, gamma)
        assert np.allclose(out[:, 0], geo, rtol=1e-13, atol=0), C
        assert np.allclose(S[0, 0], geo[-1], rtol=1e-13) and np.allclose(z[0], geo[-1], rtol=1e-13), C
        outn = o.decay_chunked(ones, ones, ones, C, gamma, True)[0]
        assert np.allclose(outn, 1.0, rtol=1e-14), C
    rng = np.random.default_rng([34, 35])
    q, k, v = _ints(rng, (12, 3)), _ints(rng, (12, 3)), _ints(rng, (12, 2))
    v2 = v.copy()
    v2[0, 1] += 4
    d = o.decay_chunked(q, k, v2, 5, 0.5)[0] - o.decay_chunked(q, k, v, 5, 0.5)[0]
    want = np.array([0.5 ** i * float(q[i] @ k[0]) * 4 for i in range(12)])
    assert np.array_equal(d[:, 1], want) and np.array_equal(d[:, 0], np.zeros(12))


def check_decay_phases(o, seed: int = 36) -> None:
    """Per-chunk states at each chunk's end, their decayed exclusive prefix, and
    the chunk output from the prefix reproduce the recurrence (exact, dyadic
    gamma on integers); the scan's total is the final state."""
    rng = np.random.default_rng([seed, 37])
    L, dk, dv = 23, 3, 2
    q, k, v = _ints(rng, (L, dk)), _ints(rng, (L, dk)), _ints(rng, (L, dv))
    g = 0.5
    ref, S, z = o.decay_state_first(q, k, v, g)
    for C in (1, 4, 6, 23, 30):
        Sn, zn, lens = o.decay_chunk_states(k, v, C, g)
        N = (L + C - 1) // C
        assert list(lens) == [min((n + 1) * C, L) - n * C for n in range(N)]
        for n in range(N):
            s, e = n * C, min((n + 1) * C, L)
            want = sum(g ** (e - 1 - j) * np.outer(k[j], v[j]) for j in range(s, e))
            assert np.array_equal(Sn[n], want), (C, n)
        P, tot = o.decay_exclusive_scan(Sn, lens, g)
        Pz, totz = o.decay_exclusive_scan(zn, lens, g)
        assert np.array_equal(tot, S) and np.array_equal(totz, z), C
        for n in range(N):
            s, e = n * C, min((n + 1) * C, L)
            rows = np.arange(e - s)
            blk = (g ** (rows + 1))[:, None] * (q[s:e] @ P[n]) + \
                ((q[s:e] @ k[s:e].T) * o.decay_weights(e - s, e - s, g)) @ v[s:e]
            assert np.array_equal(blk, ref[s:e]), (C, n)
            # the prefix is the recurrence's state after row s - 1
            Ps = o.decay_state_first(q[:s], k[:s], v[:s], g)[1] if s > 0 else np.zeros((dk, dv))
            assert np.array_equal(P[n], Ps) and np.array_equal(Pz[n], o.decay_state_first(q[:s], k[:s], v[:s], g)[2] if s > 0 else np.zeros(dk))


def check_decay_resume(o, seed: int = 38) -> None:
    """The decayed forward over L1 tokens, then decode steps from its final
    state, equals the forward over all L tokens (normalised, elu+1 features)."""
    rng = np.random.default_rng([seed, 39])
    L, L1, dk, dv = 21, 12, 3, 4
    for gamma in (0.5, 0.93):
        qf, kf, vf = o.phi_elu1(_bf16(rng, (L, dk))), o.phi_elu1(_bf16(rng, (L, dk))), _bf16(rng, (L, dv))
        full = o.decay_chunked(qf, kf, vf, 5, gamma, True)[0]
        _, S, z = o.decay_chunked(qf[:L1], kf[:L1], vf[:L1], 5, gamma, True)
        for t in range(L1, L):
            ot, S, z = o.decay_step(S, z, qf[t], kf[t], vf[t], gamma, True)
            assert np.allclose(ot, full[t], rtol=1e-12, atol=1e-14), (gamma, t)
        fullu = o.decay_chunked(qf, kf, vf, 4, gamma)[0]
        _, S, z = o.decay_chunked(qf[:L1], kf[:L1], vf[:L1], 4, gamma)
        for t in range(L1, L):
            ot, S, z = o.decay_step(S, z, qf[t], kf[t], vf[t], gamma, False)
            assert np.allclose(ot, fullu[t], rtol=1e-12, atol=1e-14), (gamma, t)


def check_decay_forward(o, seed: int = 40) -> None:
    """The forward entry point's reference with a decay: phi applied first, then
    the decayed recurrence (out, final state, final normaliser)."""
    rng = np.random.default_rng([seed, 41])
    L, dk, dv = 19, 4, 3
    q, k, v = _bf16(rng, (L, dk)), _bf16(rng, (L, dk)), _bf16(rng, (L, dv))
    for fmap, norm in (("identity", False), ("elu1", True)):
        out, S, z = o.forward(q, k, v, 5, True, norm, fmap, None, 1.0, 0.75)
        qp, kp = (q, k) if fmap == "identity" else (o.phi_elu1(q), o.phi_elu1(k))
        ref, Sr, zr = o.decay_state_first(qp, kp, v, 0.75, norm)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-14) and np.allclose(S, Sr, rtol=1e-12, atol=1e-14)
        assert np.allclose(z, zr, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Exact softmax attention (the reference of the FAVOR+ error study)
# ---------------------------------------------------------------------------
def check_softmax_reference(o, seed: int = 42) -> None:
    """softmax_attention against the term-by-term definition; its weights are a
    convex combination (outputs inside the values' range per column), the first
    causal row is v_0, a constant added to every score of a row changes nothing,
    and FAVOR+ with many orthogonal features (inputs pre-scaled by d^(-1/4)) comes
    close to it (the kernel estimate the linear-attention page derives)."""
    rng = np.random.default_rng([seed, 43])
    L, d = 9, 4
    q, k, v = rng.standard_normal((L, d)) * 0.5, rng.standard_normal((L, d)) * 0.5, rng.standard_normal((L, 3))
    for causal in (False, True):
        got = o.softmax_attention(q, k, v, causal)
        ref = np.array(o.softmax_attention_loops(q, k, v, causal))
        assert np.allclose(got, ref, rtol=1e-13, atol=1e-15), causal
    assert np.allclose(o.softmax_attention(q, k, v, True)[0], v[0], rtol=1e-15)
    out = o.softmax_attention(q, k, v)
    assert np.all(out <= v.max(axis=0) + 1e-15) and np.all(out >= v.min(axis=0) - 1e-15)
    # scores shifted by a constant: scale the queries' inner products by adding c * k-independent term
    q2 = np.concatenate([q, np.full((L, 1), 3.0)], axis=1)
    k2 = np.concatenate([k, np.ones((L, 1))], axis=1)
    assert np.allclose(o.softmax_attention(q2, k2, v, scale=1 / np.sqrt(d)), o.softmax_attention(q, k, v),
                       rtol=1e-12, atol=1e-14)
    from workloads import orthogonal_random_features
    _, W = orthogonal_random_features(65536, d, [seed, 44])
    s4 = d ** -0.25
    qp, kp = o.phi_favor(q * s4, W), o.phi_favor(k * s4, W)
    fav = (qp @ (kp.T @ v)) / (qp @ kp.sum(axis=0))[:, None]
    assert np.allclose(fav, out, rtol=0, atol=2e-2), np.abs(fav - out).max()


# ---------------------------------------------------------------------------
# Log-linear attention (the slide deck "Log-Linear Attention")
# ---------------------------------------------------------------------------
def check_loglinear_buckets(o) -> None:
    """The slides' example, t = 7: level 0 {7}, level 1 {6}, level 2 {4, 5},
    level 3 {0..3}; in general level l >= 1 holds 2^(l-1) keys, is present
    exactly when bit l-1 of t is set, and the levels partition 0..t."""
    got = {}
    for s_ in range(8):
        got.setdefault(o.loglinear_level(7, s_), []).append(s_)
    assert got == {0: [7], 1: [6], 2: [4, 5], 3: [0, 1, 2, 3]}, got
    for t in range(200):
        lev = {}
        for s_ in range(t + 1):
            lev.setdefault(o.loglinear_level(t, s_), []).append(s_)
        assert lev[0] == [t]
        for l, members in lev.items():
            if l == 0:
                continue
            assert (t >> (l - 1)) & 1, (t, l)
            h = (t >> (l - 1)) << (l - 1)
            assert members == list(range(h - (1 << (l - 1)), h)), (t, l, members)
        assert sum(len(m) for m in lev.values()) == t + 1
    assert o.loglinear_levels(1) == 1 and o.loglinear_levels(2) == 2 and o.loglinear_levels(8) == 4
    assert o.loglinear_levels(9) == 5


def check_loglinear_forms(o, seed: int = 60) -> None:
    """Integer inputs and integer weights: the masked form, the Fenwick tree
    recurrence, the chunked form at every power-of-two chunk size (1 up to past
    L) and exact brute force agree exactly; all weights 1 give linear attention;
    a weight vector that keeps one level gives that level's bucket sum."""
    rng = np.random.default_rng([seed, 61])
    L, dk, dv = 29, 3, 2
    q, k, v = _ints(rng, (L, dk)), _ints(rng, (L, dk)), _ints(rng, (L, dv))
    nl = o.loglinear_levels(L)
    lam = _ints(rng, (L, nl), -2, 3)
    ref = o.loglinear_scores_first(q, k, v, lam)
    assert np.array_equal(o.loglinear_recurrent(q, k, v, lam), ref)
    for C in (0, 1, 2, 4, 8, 16, 32, 64):
        assert np.array_equal(o.loglinear_chunked(q, k, v, lam, C), ref), C
    bf = _frac_matrix(o.brute_force_loglinear(q[:9], k[:9], v[:9], lam[:9]))
    assert np.array_equal(bf, o.loglinear_scores_first(q[:9], k[:9], v[:9], lam[:9]))
    ones = np.ones((L, nl))
    lin = o.causal_scores_first(q, k, v)
    for form in (o.loglinear_scores_first(q, k, v, ones), o.loglinear_recurrent(q, k, v, ones),
                 o.loglinear_chunked(q, k, v, ones, 8)):
        assert np.array_equal(form, lin)
    for l in range(nl):
        sel = np.zeros((L, nl))
        sel[:, l] = 1
        out = o.loglinear_chunked(q, k, v, sel, 4)
        for t in range(L):
            members = [s_ for s_ in range(t + 1) if o.loglinear_level(t, s_) == l]
            want = sum((float(q[t] @ k[s_]) * v[s_] for s_ in members), np.zeros(dv))
            assert np.array_equal(out[t], want), (l, t)


def check_loglinear_causality(o, seed: int = 62) -> None:
    """Changing token t's key or value leaves every earlier output unchanged."""
    rng = np.random.default_rng([seed, 63])
    L, d = 20, 3
    q, k, v = _ints(rng, (L, d)), _ints(rng, (L, d)), _ints(rng, (L, d))
    lam = _ints(rng, (L, o.loglinear_levels(L)), 1, 3)
    base = o.loglinear_chunked(q, k, v, lam, 4)
    for t in (0, 5, 13):
        k2, v2 = k.copy(), v.copy()
        k2[t] += 1
        v2[t] -= 2
        out = o.loglinear_chunked(q, k2, v2, lam, 4)
        assert np.array_equal(out[:t], base[:t]) and not np.array_equal(out[t:], base[t:]), t


def check_loglinear_state(o, seed: int = 64) -> None:
    """The level states the Fenwick tree recurrence leaves after token T - 1 are
    the bucket sums by definition: level l holds the sum of k_s^T v_s over the
    keys s <= T - 1 at level(T - 1, s) = l, and a level without keys is zero
    (integers: exact), for every T up to L."""
    rng = np.random.default_rng([seed, 65])
    L, dk, dv = 37, 3, 2
    q, k, v = _ints(rng, (L, dk)), _ints(rng, (L, dk)), _ints(rng, (L, dv))
    nl = o.loglinear_levels(L)
    lam = _ints(rng, (L, nl), -2, 3)
    for T in range(1, L + 1):
        _, S = o.loglinear_recurrent(q[:T], k[:T], v[:T], lam[:T], return_state=True)
        assert S.shape == (nl, dk, dv)
        for l in range(nl):
            want = np.zeros((dk, dv))
            for s_ in range(T):
                if o.loglinear_level(T - 1, s_) == l:
                    want += np.outer(k[s_], v[s_]).astype(np.float64)
            assert np.array_equal(S[l], want), (T, l)


def check_loglinear_resume(o, seed: int = 66) -> None:
    """Running the recurrence to token T0 - 1, then on from its state at token
    T0, gives the uninterrupted run's outputs and final state (integers:
    exact), for split points on and between powers of two."""
    rng = np.random.default_rng([seed, 67])
    L, dk, dv = 70, 3, 2
    q, k, v = _ints(rng, (L, dk)), _ints(rng, (L, dk)), _ints(rng, (L, dv))
    lam = _ints(rng, (L, o.loglinear_levels(L)), -2, 3)
    full, S_full = o.loglinear_recurrent(q, k, v, lam, return_state=True)
    for T0 in (1, 2, 7, 8, 31, 32, 33, 64, 69):
        a, S_a = o.loglinear_recurrent(q[:T0], k[:T0], v[:T0], lam[:T0], return_state=True)
        b, S_b = o.loglinear_recurrent(q[T0:], k[T0:], v[T0:], lam[T0:], S0=S_a, t0=T0, return_state=True)
        assert np.array_equal(np.concatenate([a, b]), full), T0
        assert np.array_equal(S_b, S_full), T0


# ---------------------------------------------------------------------------
# The forward's reference: phi of the scaled inputs, and its non-causal branch
# ---------------------------------------------------------------------------
def check_apply_phi_in_scale(o) -> None:
    """apply_phi(x, f, W, s) is phi(s x): the scale multiplies the input before the
    map (linear-attention page: the Performer implementation scales Q and K by
    d^(-1/4) before FAVOR+).  Hand-computed points: elu+1 at s = -0.5 and s = 1/4
    (s x = -1 -> e^-1, s x = 0.5 -> 1.5, ...), the identity at s = 3, FAVOR+ at
    s = 1/2 with a hand-written W."""
    x = np.array([2.0, -1.0, 0.5, 0.0, -4.0])
    cases = {
        -0.5: [math.exp(-1.0), 1.5, math.exp(-0.25), 1.0, 3.0],   # s x = -1, 0.5, -0.25, 0, 2
        0.25: [1.5, math.exp(-0.25), 1.125, 1.0, math.exp(-1.0)],  # s x = 0.5, -0.25, 0.125, 0, -1
    }
    for s, want in cases.items():
        assert np.allclose(o.apply_phi(x, "elu1", None, s), want, rtol=1e-15, atol=0), s
    assert np.array_equal(o.apply_phi(x, "identity", None, 3.0), 3.0 * x)
    W = np.array([[1.0, 0, 0], [0, 1.0, 0], [0, 0, 1.0], [1.0, -1.0, 2.0]])
    xf = np.array([1.0, 2.0, -1.0])
    # s x = [0.5, 1, -0.5]: |s x|^2 / 2 = 0.75; projections 0.5, 1, -0.5, -1.5; m = 4
    want = np.array([math.exp(-0.25), math.exp(0.25), math.exp(-1.25), math.exp(-2.25)]) / 2.0
    assert np.allclose(o.apply_phi(xf, "favor", W, 0.5), want, rtol=1e-15, atol=0)
    assert np.allclose(o.apply_phi(xf[None, :], "favor", W, 0.5)[0], want, rtol=1e-15, atol=0)


def check_forward_scaled_favor_is_softmax(o, seed: int = 46) -> None:
    """forward(..., fmap="favor", in_scale=d^(-1/4)) with many orthogonal features
    approaches softmax(q k^T / sqrt(d)) v, causal and not (the linear-attention
    page's Performer: FAVOR+ of the pre-scaled inputs estimates exp(q.k/sqrt(d)),
    so the normalised ratio estimates softmax attention).  Without the scale it
    estimates softmax at scale 1 instead, which the same check tells apart."""
    from workloads import orthogonal_random_features
    rng = np.random.default_rng([seed, 47])
    L, d = 8, 4
    q, k = rng.standard_normal((L, d)) * 0.9, rng.standard_normal((L, d)) * 0.9
    v = rng.standard_normal((L, 3))
    _, W = orthogonal_random_features(65536, d, [seed, 48])
    s4 = d ** -0.25
    for causal in (False, True):
        out = o.forward(q, k, v, 3, causal, True, "favor", W, s4)[0]
        ref = o.softmax_attention(q, k, v, causal)
        assert np.allclose(out, ref, rtol=0, atol=2e-2), (causal, np.abs(out - ref).max())
        other = o.softmax_attention(q, k, v, causal, scale=1.0)
        assert np.abs(other - ref).max() > 0.1  # the scale is visible at this tolerance


def check_forward_noncausal(o, seed: int = 49) -> None:
    """forward(causal=False) against exact brute force over all keys, with and
    without the normaliser, for the identity (integers, exact) and elu+1 (bf16
    values), and its final state = sum_t phi(k_t)^T v_t, z = sum_t phi(k_t)
    (chunking page, section ①; linear-attention page, normalised output).  The
    chunk size is ignored."""
    rng = np.random.default_rng([seed, 50])
    L, dk, dv = 7, 3, 2
    q, k, v = _ints(rng, (L, dk)), _ints(rng, (L, dk)), _ints(rng, (L, dv))
    for C in (1, 3, 7):
        out, S, z = o.forward(q, k, v, C, False, False)
        bf = np.array([[int(x) for x in row] for row in o.brute_force(q, k, v, causal=False)], dtype=np.int64)
        assert np.array_equal(np.asarray(out), bf), C
        S_def = sum(np.outer(k[t], v[t]) for t in range(L))
        assert np.array_equal(S, S_def) and np.array_equal(z, k.sum(axis=0))
    qf, kf, vf = _bf16(rng, (L, dk)), _bf16(rng, (L, dk)), _bf16(rng, (L, dv))
    qp, kp = o.phi_elu1(qf), o.phi_elu1(kf)
    for normalize in (False, True):
        out, S, z = o.forward(qf, kf, vf, 2, False, normalize, "elu1")
        exact = _frac_matrix(o.brute_force(qp, kp, vf, causal=False, normalize=normalize))
        assert np.allclose(out, exact, rtol=1e-12, atol=1e-13), normalize
        assert np.allclose(S, sum(np.outer(kp[t], vf[t]) for t in range(L)), rtol=1e-13, atol=1e-14)
        assert np.allclose(z, kp.sum(axis=0), rtol=1e-13, atol=1e-14)
    # the identity with a scale s: s q, s k, so the unnormalised output is s^2 times
    out = o.forward(q, k, v, 3, False, False, "identity", None, 2.0)[0]
    assert np.array_equal(out, 4.0 * np.asarray(o.forward(q, k, v, 3, False, False)[0], dtype=np.float64))
    # with a scale: phi(s q), phi(s k) (s < 0 flips which branch of elu+1 applies)
    out = o.forward(qf, kf, vf, 2, False, True, "elu1", None, -0.5)[0]
    qs, ks = o.phi_elu1(-0.5 * qf), o.phi_elu1(-0.5 * kf)
    exact = _frac_matrix(o.brute_force(qs, ks, vf, causal=False, normalize=True))
    assert np.allclose(out, exact, rtol=1e-12, atol=1e-13)


def check_forward_causal_scaled(o, seed: int = 51) -> None:
    """forward(causal=True) with a map and a scale against exact brute force on
    phi(s q), phi(s k), for every chunk size (chunking page, section ②)."""
    rng = np.random.default_rng([seed, 52])
    L, dk, dv = 9, 3, 2
    qf, kf, vf = _bf16(rng, (L, dk)), _bf16(rng, (L, dk)), _bf16(rng, (L, dv))
    for s in (0.5, -2.0):
        qs, ks = o.phi_elu1(s * qf), o.phi_elu1(s * kf)
        for normalize in (False, True):
            exact = _frac_matrix(o.brute_force(qs, ks, vf, causal=True, normalize=normalize))
            for C in (1, 4, 9):
                out, S, z = o.forward(qf, kf, vf, C, True, normalize, "elu1", None, s)
                assert np.allclose(out, exact, rtol=1e-12, atol=1e-13), (s, normalize, C)
                assert np.allclose(S, ks.T @ vf, rtol=1e-13, atol=1e-14)


def check_over_heads(o, seed: int = 53) -> None:
    """over_heads maps a single-head form over a leading head axis: head h of the
    result is the form on head h alone, for forms returning one array or a tuple."""
    rng = np.random.default_rng([seed, 54])
    H, L, dk, dv = 3, 6, 2, 3
    q, k, v = _ints(rng, (H, L, dk)), _ints(rng, (H, L, dk)), _ints(rng, (H, L, dv))
    one = o.over_heads(o.causal_scores_first, q, k, v)
    tup = o.over_heads(o.chunked, q, k, v, 4)
    assert one.shape == (H, L, dv) and len(tup) == 3 and tup[1].shape == (H, dk, dv)
    for h in range(H):
        assert np.array_equal(one[h], o.causal_scores_first(q[h], k[h], v[h]))
        out, S, z = o.chunked(q[h], k[h], v[h], 4)
        assert np.array_equal(tup[0][h], out) and np.array_equal(tup[1][h], S) and np.array_equal(tup[2][h], z)


# ---------------------------------------------------------------------------
# The delta rule (Kimi/Qwen page "Kimi K3 と Qwen 3.8 の Attention 機構比較分析":
# section 3.1, the erase-then-write update of its equation (14); section 2.4,
# the gated form; section 3.3.5, the two-key example).  The recurrence is the
# definition; every other form is pinned to it, to exact brute force, to the
# page's worked example and to cases that reduce to forms pinned above.
# ---------------------------------------------------------------------------
def _frac_rows(rows):
    return np.array([[float(x) for x in r] for r in rows])


def check_delta_page_example(o) -> None:
    """Section 3.3.5: unit keys k1 = [1, 0], k2 = [cos t, sin t]; write v1 under k1,
    then v2 under k2 (full strength); reading with k1 gives sin^2 t v1 + cos t v2.
    Exact with cos t = 3/5, sin t = 4/5; the page's cos t = 0.98 leaves 0.98 of v2
    and 1 - 0.98^2 = 0.0396 of v1."""
    F = Fraction
    v1, v2 = [F(2), F(-1), F(5)], [F(1), F(3), F(-2)]
    k = [[F(1), F(0)], [F(3, 5), F(4, 5)]]
    q = [[F(0), F(0)], [F(1), F(0)]]  # the second read is with k1
    out, S = o.brute_force_delta(q, k, [v1, v2], [F(1), F(1)])
    want = [F(16, 25) * a + F(3, 5) * b for a, b in zip(v1, v2)]
    assert out[1] == want, (out[1], want)
    c = 0.98
    s_ = math.sqrt(1 - c * c)
    kf = np.array([[1.0, 0.0], [c, s_]])
    vf = np.array([[2.0, -1.0, 5.0], [1.0, 3.0, -2.0]])
    qf = np.array([[0.0, 0.0], [1.0, 0.0]])
    for form in (lambda: o.delta_recurrent(qf, kf, vf, [1.0, 1.0])[0],
                 lambda: o.delta_chunked(qf, kf, vf, [1.0, 1.0], None, 2)[0]):
        got = form()[1]
        assert np.allclose(got, (1 - c * c) * vf[0] + c * vf[1], rtol=1e-13, atol=1e-14), got
    assert abs((1 - c * c) - 0.0396) < 1e-15


def check_delta_readback(o, seed: int = 70) -> None:
    """Equation (14) of section 3.1: the old prediction at the key is erased and
    the new value written, so right after a full-strength write under a unit key
    the state maps that key exactly to the new value, whatever it held before;
    and a key written twice returns the second value (section 3.3.6: the last
    write wins).  Exact on Fractions with unit keys e_i and (3/5, 4/5)."""
    rng = np.random.default_rng([seed, 71])
    F = Fraction
    dk, dv = 3, 2
    units = [[F(1), F(0), F(0)], [F(0), F(3, 5), F(4, 5)], [F(4, 5), F(0), F(-3, 5)], [F(0), F(1), F(0)]]
    L = 7
    ks = [units[i % 4] for i in rng.permutation(L)]
    ks[5] = ks[2]  # the same key twice
    vs = [[F(int(x)) for x in rng.integers(-4, 5, dv)] for _ in range(L)]
    # queries equal to the keys: each read-back must return the value just written
    out, S = o.brute_force_delta(ks, ks, vs, [F(1)] * L)
    for t in range(L):
        assert out[t] == vs[t], t
    # from a nonzero state, through the float forms (keys exact in binary: e_i only)
    S0 = rng.integers(-3, 4, (dk, dv)).astype(np.float64)
    kf = np.eye(dk)[rng.integers(0, dk, L)]
    vf = rng.integers(-4, 5, (L, dv)).astype(np.float64)
    for form in (o.delta_recurrent(kf, kf, vf, np.ones(L), None, S0)[0],
                 o.delta_chunked(kf, kf, vf, np.ones(L), None, 3, S0)[0]):
        assert np.array_equal(form, vf)


def check_delta_orthogonal_keys(o, seed: int = 72) -> None:
    """With keys orthogonal to every earlier key the erase finds nothing: u_t =
    beta_t v_t, so the delta rule is causal linear attention on values beta_t v_t,
    and with a constant gate gamma the decayed (Retention) recurrence; both pinned
    above.  Exact on integers and dyadic beta, gamma."""
    rng = np.random.default_rng([seed, 73])
    L = dk = 6
    dv = 3
    k = np.eye(dk)[rng.permutation(dk)] * rng.choice([-1.0, 1.0], (L, 1))
    q = rng.integers(-3, 4, (L, dk)).astype(np.float64)
    v = rng.integers(-3, 4, (L, dv)).astype(np.float64)
    b = rng.choice([0.25, 0.5, 1.0], L)
    ref = o.causal_scores_first(q, k, b[:, None] * v)
    for C in (1, 2, 4, 6):
        assert np.array_equal(o.delta_chunked(q, k, v, b, None, C)[0], ref), C
    assert np.array_equal(o.delta_recurrent(q, k, v, b)[0], ref)
    gam = 0.75
    refd, Sd, _ = o.decay_state_first(q, k, b[:, None] * v, gam)
    for C in (1, 3, 6):
        out, S = o.delta_chunked(q, k, v, b, np.full(L, gam), C)
        assert np.array_equal(out, refd) and np.array_equal(S, Sd), C


def check_delta_scalar_closed_form(o) -> None:
    """d_k = 1 with the key 1: S_t = alpha_t (1 - beta) S_{t-1} + beta v_t, an
    exponential moving average; with alpha = 1 and S_0 = 0,
    S_t = sum_{j<=t} beta (1 - beta)^(t-j) v_j, so the two write orders of two
    values differ by beta^2 (v_2 - v_1) (section 3.3.6: the update does not
    commute), and beta = 1 keeps only the last value.  beta = 0 leaves the
    state to the gates: S_t = (prod of alpha) S_0."""
    v = np.array([[3.0], [-5.0], [7.0], [1.0]])
    one = np.ones((4, 1))
    for beta in (0.5, 0.25, 1.0):
        out = o.delta_recurrent(one, one, v, np.full(4, beta))[0]
        for t in range(4):
            want = sum(beta * (1 - beta) ** (t - j) * v[j, 0] for j in range(t + 1))
            assert out[t, 0] == want, (beta, t)
        a = o.delta_chunked(one[:2], one[:2], v[:2], [beta, beta], None, 2)[0][1, 0]
        b_ = o.delta_chunked(one[:2], one[:2], v[1::-1], [beta, beta], None, 2)[0][1, 0]
        assert a - b_ == beta * beta * (v[1, 0] - v[0, 0])
    alpha = np.array([0.5, 0.75, 1.0, 0.5])
    S0 = np.array([[8.0, -4.0]])
    for form in (o.delta_recurrent(one, one, np.zeros((4, 2)), np.zeros(4), alpha, S0),
                 o.delta_chunked(one, one, np.zeros((4, 2)), np.zeros(4), alpha, 3, S0)):
        out, S = form
        assert np.array_equal(out[:, 0], 8.0 * np.cumprod(alpha)) and np.array_equal(S, S0 * np.prod(alpha))


def check_delta_forms(o, seed: int = 74) -> None:
    """The chunked form equals the recurrence for every chunk size: exactly on
    integers at full strength without gates (the triangular system is integer);
    with fractional beta and gates against exact brute force to float64
    rounding; and the recurrence against brute force."""
    rng = np.random.default_rng([seed, 75])
    L, dk, dv = 9, 3, 2
    q, k, v = (rng.integers(-1, 2, (L, d)).astype(np.float64) for d in (dk, dk, dv))
    ref, S = o.delta_recurrent(q, k, v, np.ones(L))
    bf, Sb = o.brute_force_delta(q, k, v, np.ones(L))
    assert np.array_equal(ref, _frac_rows(bf)) and np.array_equal(S, _frac_rows(Sb))
    for C in range(0, L + 2):
        out, Sc = o.delta_chunked(q, k, v, np.ones(L), None, C)
        assert np.array_equal(out, ref) and np.array_equal(Sc, S), C
    qf, kf, vf = _bf16(rng, (L, dk)), _bf16(rng, (L, dk), 0.6), _bf16(rng, (L, dv))
    b = rng.choice([0.25, 0.5, 0.75, 1.0], L)
    a = rng.choice([0.5, 0.75, 1.0], L)
    bf, Sb = o.brute_force_delta(qf, kf, vf, b, a)
    exact, Sx = _frac_rows(bf), _frac_rows(Sb)
    r, Sr = o.delta_recurrent(qf, kf, vf, b, a)
    assert np.allclose(r, exact, rtol=1e-12, atol=1e-13) and np.allclose(Sr, Sx, rtol=1e-12, atol=1e-13)
    for C in (1, 2, 4, 5, 9, 12):
        out, Sc = o.delta_chunked(qf, kf, vf, b, a, C)
        assert np.allclose(out, exact, rtol=1e-12, atol=1e-13), C
        assert np.allclose(Sc, Sx, rtol=1e-12, atol=1e-13), C


def check_delta_transform(o, seed: int = 76) -> None:
    """The chunk transform T = (I + A)^(-1) diag(beta), A[i, j] = beta_i (k_i.k_j)
    g_i / g_j (j < i): lower triangular with diagonal beta, (I + A) T = diag(beta)
    exactly on integer keys, and for the first chunk (zero state) the outputs
    are (tril(Q K^T) * G) T V, the recurrence's first rows."""
    rng = np.random.default_rng([seed, 77])
    L, dk, dv, C = 11, 3, 2, 5
    k = rng.integers(-1, 2, (L, dk)).astype(np.float64)
    Ts = o.delta_chunk_transform(k, np.ones(L), None, C)
    assert [t.shape for t in Ts] == [(5, 5), (5, 5), (1, 1)]
    for n, T in enumerate(Ts):
        kc = k[n * C:(n + 1) * C]
        A = np.tril(kc @ kc.T, -1)
        assert np.array_equal((np.eye(len(kc)) + A) @ T, np.eye(len(kc)))
        assert np.array_equal(np.triu(T, 1), np.zeros_like(T))
    qf, kf, vf = _bf16(rng, (C, dk)), _bf16(rng, (C, dk), 0.6), _bf16(rng, (C, dv))
    b = rng.choice([0.25, 0.5, 1.0], C)
    a = rng.choice([0.5, 0.75, 1.0], C)
    T = o.delta_chunk_transform(kf, b, a, C)[0]
    assert np.allclose(np.diag(T), b, rtol=1e-15)
    g = np.cumprod(a)
    out0 = (np.tril(qf @ kf.T) * (g[:, None] / g[None, :])) @ T @ vf
    assert np.allclose(out0, o.delta_recurrent(qf, kf, vf, b, a)[0], rtol=1e-12, atol=1e-13)


def check_delta_causality_resume(o, seed: int = 78) -> None:
    """Changing token t changes no earlier output; the chunked form over the
    first L1 tokens followed by decode steps from its final state equals the
    form over all L tokens."""
    rng = np.random.default_rng([seed, 79])
    L, L1, dk, dv = 14, 9, 4, 3
    q, k, v = _bf16(rng, (L, dk)), _bf16(rng, (L, dk), 0.5), _bf16(rng, (L, dv))
    b, a = rng.uniform(0.1, 1.0, L), rng.uniform(0.6, 1.0, L)
    base, Sfull = o.delta_chunked(q, k, v, b, a, 4)
    for t in (0, 5, 8, 13):
        for which in range(3):
            arrs = [q.copy(), k.copy(), v.copy()]
            arrs[which][t] += 0.5
            pert = o.delta_chunked(*arrs, b, a, 4)[0]
            assert np.array_equal(pert[:t], base[:t]), (t, which)
            assert not np.allclose(pert[t:], base[t:]), (t, which)
    _, S = o.delta_chunked(q[:L1], k[:L1], v[:L1], b[:L1], a[:L1], 4)
    for t in range(L1, L):
        ot, S = o.delta_step(S, q[t], k[t], v[t], b[t], a[t])
        assert np.allclose(ot, base[t], rtol=1e-12, atol=1e-13), t
    assert np.allclose(S, Sfull, rtol=1e-12, atol=1e-13)
