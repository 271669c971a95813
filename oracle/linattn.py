"""CPU oracle for chunkwise-parallel causal linear attention.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP path (``chunked_causal_linear_amd``) and imports nothing
from it.

Everything here is the plain definition of what the method computes, written
from four pages:

* "attention と線形の間" (sharin-2a1.pages.dev/parts/chunked.html), below
  called *the chunking page*: section ① (the two association orders and the
  d x d state), section ② (the chunked algorithm and its two causal ends) and
  section ③ (the operation counts).
* the slide deck "Log-Linear Attention" (docswell): the Fenwick-tree token
  partition, the hierarchical mask, its recurrence and chunkwise computation.
* "Linear Attention / Performerの理論と実装" (disassemble-channel.com/
  linear-attention/), below called *the linear-attention page*: the kernel
  re-formulation with feature maps and normaliser, the RNN view (state S_t,
  normaliser z_t, and the decayed recurrence it gives for Retention), the
  elu+1 and FAVOR+ feature maps, and the recurrent and materialised-prefix
  causal forms.
* "Kimi K3 と Qwen 3.8 の Attention 機構比較分析" (news.ainew.jp), below called
  *the Kimi/Qwen page*: the delta rule's erase-then-write update (section 3.1),
  its gated form (section 2.4) and its two-key example (section 3.3.5).

Precision.  Floating-point inputs arrive as float64 arrays holding bf16 values
(exact), and every form computes in float64 with no intermediate rounding.
Integer inputs arrive as int64 arrays; the matrix forms then compute in float64,
which is exact because every intermediate is an integer below 2**53 in
magnitude (``_check_int_exact`` asserts the bound), and the results are returned
as int64.  ``brute_force`` uses Python integers / Fractions and pins the rest.

Shapes.  All forms take one head: q, k as [L, d_k] (after the feature map),
v as [L, d_v].  ``over_heads`` maps a form over a leading head axis.

Parity status.  Every function below is pinned by tests under
``tests/test_oracle_*.py`` (closed forms, brute force, exhaustive tiny cases,
cross-form identities, the chunking page's printed tables); ``apply_phi`` and
``forward`` at hand-computed points of phi(s x), against brute force on both
causal ends and with the scale, and against softmax attention for FAVOR+ with
the d^(-1/4) scale.  ``phi_favor`` is
pinned by its closed form at hand-computed points and by the large-m
convergence of phi(q).phi(k) to exp(q.k); the W it consumes is an input.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Callable, Optional, Tuple

import numpy as np

_EXACT_LIMIT = 2 ** 53


# ---------------------------------------------------------------------------
# Feature maps (linear-attention page: ELU feature map, FAVOR+ positive random
# features).  The map is applied to queries and keys only, never to values.
# ---------------------------------------------------------------------------
def phi_identity(x: np.ndarray) -> np.ndarray:
    """No feature map: the chunking page works directly on q and k."""
    return x


def phi_elu1(x: np.ndarray) -> np.ndarray:
    """elu(x) + 1 with ELU's alpha = 1: x + 1 where x >= 0, exp(x) where x < 0."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x >= 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def phi_favor(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """FAVOR+ positive random features.

    phi(x)_l = exp(w_l . x - |x|^2 / 2) / sqrt(m) for the m rows w_l of W
    (linear-attention page, FAVOR+ section: positive random features and their
    implementation).  x: [..., d], W: [m, d] -> [..., m].
    """
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    m = W.shape[0]
    proj = x @ W.T
    half_sq = 0.5 * np.sum(x * x, axis=-1, keepdims=True)
    return np.exp(proj - half_sq) / np.sqrt(m)


def apply_phi(x: np.ndarray, fmap: str, W: Optional[np.ndarray] = None,
              in_scale: float = 1.0) -> np.ndarray:
    """phi(in_scale * x) for fmap in {"identity", "elu1", "favor"}."""
    if in_scale != 1.0:
        x = np.asarray(x, dtype=np.float64) * in_scale
    if fmap == "identity":
        return phi_identity(x)
    if fmap == "elu1":
        return phi_elu1(x)
    if fmap == "favor":
        if W is None:
            raise ValueError("favor needs W")
        return phi_favor(x, W)
    raise ValueError(fmap)


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------
def _is_int(*arrays) -> bool:
    return all(np.issubdtype(np.asarray(a).dtype, np.integer) for a in arrays)


def _check_int_exact(q, k, v) -> None:
    """Integer inputs: the float64 matrix forms are exact below 2**53.

    Any entry of any intermediate is bounded by L * d_k * max|q| * max|k| * max|v|
    (scores times values, or queries times the summed state).
    """
    L, dk = q.shape
    bound = (L * dk * max(1, int(np.abs(q).max(initial=0))) * max(1, int(np.abs(k).max(initial=0)))
             * max(1, int(np.abs(v).max(initial=0))))
    if bound >= _EXACT_LIMIT:
        raise OverflowError("integer case too large for exact float64 evaluation")


def _prep(q, k, v):
    integer = _is_int(q, k, v)
    if integer:
        _check_int_exact(np.asarray(q), np.asarray(k), np.asarray(v))
    return (np.asarray(q, dtype=np.float64), np.asarray(k, dtype=np.float64),
            np.asarray(v, dtype=np.float64), integer)


def _finish(x: np.ndarray, integer: bool) -> np.ndarray:
    if integer:
        r = np.rint(x)
        assert np.array_equal(r, x), "non-integer intermediate on the integer path"
        return r.astype(np.int64)
    return x


def tril(scores: np.ndarray) -> np.ndarray:
    """Causal mask: zero position (i, j) for j > i, keep the diagonal.

    The chunking page's tril keeps j <= i (a token sees itself); the RNN view of
    the linear-attention page adds token t to the state before reading it.
    """
    n_rows, n_cols = scores.shape[-2], scores.shape[-1]
    keep = np.arange(n_cols)[None, :] <= np.arange(n_rows)[:, None]
    return np.where(keep, scores, 0.0)


def _divide(num: np.ndarray, den: np.ndarray) -> np.ndarray:
    """Row-wise division of the numerator by the denominator, no epsilon."""
    with np.errstate(divide="ignore", invalid="ignore"):
        return num / den[..., None]


# ---------------------------------------------------------------------------
# O1: causal scores-first  (chunking page, section ②: CausalScoresFirst;
# linear-attention page: normalised output as a ratio of kernel sums)
# ---------------------------------------------------------------------------
def causal_scores_first(q, k, v, normalize: bool = False) -> np.ndarray:
    """A = tril(q k^T) (L x L); numerator A v; normalised: divide by the row sums of A."""
    q, k, v, integer = _prep(q, k, v)
    A = tril(q @ k.T)
    num = A @ v
    if not normalize:
        return _finish(num, integer)
    return _divide(num, A.sum(axis=1))


# ---------------------------------------------------------------------------
# O2: causal state-first, token by token (chunking page, section ②:
# CausalStateFirst; linear-attention page: RNN view, S_t and z_t recurrences)
# ---------------------------------------------------------------------------
def causal_state_first(q, k, v, normalize: bool = False, S0=None, z0=None):
    """S_t = S_{t-1} + k_t^T v_t, z_t = z_{t-1} + k_t; read y_t = q_t S_t [/ q_t . z_t].

    The state is updated with token t before token t reads it.  Returns
    (out [L, d_v], S_L [d_k, d_v], z_L [d_k]).  S0/z0 continue from a given state
    (zero when omitted, as on both pages).
    """
    q, k, v, integer = _prep(q, k, v)
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    z = np.zeros(dk) if z0 is None else np.array(z0, dtype=np.float64)
    out = np.zeros((L, dv))
    for t in range(L):
        S = S + np.outer(k[t], v[t])
        z = z + k[t]
        num = q[t] @ S
        out[t] = num / (q[t] @ z) if normalize else num
    if normalize:
        return out, S, z
    return _finish(out, integer), _finish(S, integer), _finish(z, integer)


def recurrent_step(S, z, q_t, k_t, v_t, normalize: bool = True):
    """One decode step on one state: S += k^T v, z += k, then o = q S [/ q . z].

    The same update-then-read order as causal_state_first.  Returns (o, S', z').
    """
    S = np.asarray(S, dtype=np.float64) + np.outer(k_t, v_t)
    z = np.asarray(z, dtype=np.float64) + k_t
    num = q_t @ S
    o = num / (q_t @ z) if normalize else num
    return o, S, z


# ---------------------------------------------------------------------------
# O2': the materialised-prefix causal form (linear-attention page: the
# "parallel" causal implementation that stores every prefix state)
# ---------------------------------------------------------------------------
def causal_materialized_prefix(q, k, v, normalize: bool = False) -> np.ndarray:
    """Store all L prefix states S_1..S_L (L x d_k x d_v) first, then read each."""
    q, k, v, integer = _prep(q, k, v)
    S_pref = np.cumsum(k[:, :, None] * v[:, None, :], axis=0)
    z_pref = np.cumsum(k, axis=0)
    num = np.einsum("ta,tab->tb", q, S_pref)
    if not normalize:
        return _finish(num, integer)
    return _divide(num, np.einsum("ta,ta->t", q, z_pref))


# ---------------------------------------------------------------------------
# O3: chunked (chunking page, section ②: Chunked), with the normaliser of the
# linear-attention page carried alongside the state.
# ---------------------------------------------------------------------------
def chunked(q, k, v, C: int, normalize: bool = False):
    """Chunkwise form with chunk size C (C <= 0 is treated as 1).

    State starts at zero.  For each chunk [s, e) (the last may be shorter):
        inter = q_c state            (and q_c . z for the denominator)
        intra = tril(q_c k_c^T) v_c  (and the row sums of tril(q_c k_c^T))
        out_c = inter + intra        (normalised: numerator / denominator)
        state += k_c^T v_c ; z += sum of k_c rows
    Returns (out, S_L, z_L).
    """
    if C <= 0:
        C = 1
    q, k, v, integer = _prep(q, k, v)
    L, dk = q.shape
    dv = v.shape[1]
    out = np.zeros((L, dv))
    S = np.zeros((dk, dv))
    z = np.zeros(dk)
    for s in range(0, L, C):
        e = min(s + C, L)
        qc, kc, vc = q[s:e], k[s:e], v[s:e]
        sc = tril(qc @ kc.T)
        num = qc @ S + sc @ vc
        if normalize:
            den = qc @ z + sc.sum(axis=1)
            out[s:e] = _divide(num, den)
        else:
            out[s:e] = num
        S = S + kc.T @ vc
        z = z + kc.sum(axis=0)
    if normalize:
        return out, S, z
    return _finish(out, integer), _finish(S, integer), _finish(z, integer)


# ---------------------------------------------------------------------------
# Phase definitions used by the three-kernel pipeline: per-chunk states and
# their exclusive prefix (chunking page, section ②: the state carried across
# chunks is the sum of k_c^T v_c over the chunks already processed).
# ---------------------------------------------------------------------------
def chunk_states(k, v, C: int):
    """Per-chunk local states S_n = k_c^T v_c and z_n = sum of k_c rows, n = 0..N-1."""
    if C <= 0:
        C = 1
    integer = _is_int(k, v)
    kf = np.asarray(k, dtype=np.float64)
    vf = np.asarray(v, dtype=np.float64)
    L, dk = kf.shape
    N = (L + C - 1) // C
    S = np.zeros((N, dk, vf.shape[1]))
    z = np.zeros((N, dk))
    for n in range(N):
        s, e = n * C, min((n + 1) * C, L)
        S[n] = kf[s:e].T @ vf[s:e]
        z[n] = kf[s:e].sum(axis=0)
    return _finish(S, integer), _finish(z, integer)


def exclusive_scan(S_n: np.ndarray):
    """P_0 = 0, P_n = P_{n-1} + S_{n-1}; also the total sum (the final state)."""
    integer = _is_int(S_n)
    Sf = np.asarray(S_n, dtype=np.float64)
    P = np.zeros_like(Sf)
    run = np.zeros(Sf.shape[1:])
    for n in range(Sf.shape[0]):
        P[n] = run
        run = run + Sf[n]
    return _finish(P, integer), _finish(run, integer)


# ---------------------------------------------------------------------------
# O4: non-causal, both association orders (chunking page, section ①:
# ScoresFirst, StateFirst, State; linear-attention page: matrix form with the
# diag^{-1} normaliser and its linear_attention description)
# ---------------------------------------------------------------------------
def noncausal_scores_first(q, k, v, normalize: bool = False) -> np.ndarray:
    q, k, v, integer = _prep(q, k, v)
    A = q @ k.T
    if not normalize:
        return _finish(A @ v, integer)
    return _divide(A @ v, A.sum(axis=1))


def noncausal_state_first(q, k, v, normalize: bool = False) -> np.ndarray:
    q, k, v, integer = _prep(q, k, v)
    S = k.T @ v
    if not normalize:
        return _finish(q @ S, integer)
    return _divide(q @ S, q @ k.sum(axis=0))


def final_state(k, v):
    """S = sum_t k_t^T v_t (d_k x d_v, independent of L) and z = sum_t k_t."""
    integer = _is_int(k, v)
    kf = np.asarray(k, dtype=np.float64)
    vf = np.asarray(v, dtype=np.float64)
    return _finish(kf.T @ vf, integer), _finish(kf.sum(axis=0), integer)


# ---------------------------------------------------------------------------
# O7: brute force on tiny inputs, in exact arithmetic
# ---------------------------------------------------------------------------
def brute_force(q, k, v, causal: bool = True, normalize: bool = False):
    """o_{i,c} = sum_{j<=i} sum_a q_{i,a} k_{j,a} v_{j,c}  [/ sum_{j<=i} sum_a q_{i,a} k_{j,a}].

    Nested Python loops over exact integers (or Fractions of the exact binary
    values of float inputs).  Returns a list of lists of Fractions.
    """
    def exact(x):
        if isinstance(x, (int, np.integer)):
            return Fraction(int(x))
        return Fraction(float(x))

    L, dk = len(q), len(q[0])
    dv = len(v[0])
    out = []
    for i in range(L):
        last = i if causal else L - 1
        row = []
        den = Fraction(0)
        for j in range(last + 1):
            for a in range(dk):
                den += exact(q[i][a]) * exact(k[j][a])
        for c in range(dv):
            acc = Fraction(0)
            for j in range(last + 1):
                s = Fraction(0)
                for a in range(dk):
                    s += exact(q[i][a]) * exact(k[j][a])
                acc += s * exact(v[j][c])
            row.append(acc / den if normalize else acc)
        out.append(row)
    return out


# ---------------------------------------------------------------------------
# Retention decay (linear-attention page, RNN view, where forgetting is
# introduced: S_t = gamma S_{t-1} + phi(k_t) v_t^T with 0 < gamma < 1).  The page
# gives the state recurrence only; the normaliser is read as decaying the same
# way, z_t = gamma z_{t-1} + phi(k_t), and the read stays y_t = phi(q_t) S_t
# [/ phi(q_t) . z_t] after the update.  gamma = 1 is plain linear attention.
# All of these compute in float64 (the decay weights are not integers).
# ---------------------------------------------------------------------------
def _f64(*arrays):
    return tuple(np.asarray(a, dtype=np.float64) for a in arrays)


def decay_weights(n_rows: int, n_cols: int, gamma: float) -> np.ndarray:
    """D[i, j] = gamma^(i - j) where j <= i, else 0: the weight with which key j
    reaches the read of query i (unrolling the recurrence i - j times)."""
    e = np.arange(n_rows)[:, None] - np.arange(n_cols)[None, :]
    return np.where(e >= 0, float(gamma) ** np.maximum(e, 0), 0.0)


def decay_state_first(q, k, v, gamma: float, normalize: bool = False, S0=None, z0=None):
    """The recurrence itself, token by token: S_t = gamma S_{t-1} + k_t^T v_t,
    z_t = gamma z_{t-1} + k_t, then y_t = q_t S_t [/ q_t . z_t].  Returns
    (out, S_L, z_L); S0/z0 continue from a given state (zero when omitted)."""
    q, k, v = _f64(q, k, v)
    L, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    z = np.zeros(dk) if z0 is None else np.array(z0, dtype=np.float64)
    out = np.zeros((L, dv))
    for t in range(L):
        S = gamma * S + np.outer(k[t], v[t])
        z = gamma * z + k[t]
        num = q[t] @ S
        out[t] = num / (q[t] @ z) if normalize else num
    return out, S, z


def decay_step(S, z, q_t, k_t, v_t, gamma: float, normalize: bool = True):
    """One decode step of the decayed recurrence: S = gamma S + k^T v, z = gamma z
    + k, then o = q S [/ q . z].  Returns (o, S', z')."""
    S = gamma * np.asarray(S, dtype=np.float64) + np.outer(k_t, v_t)
    z = gamma * np.asarray(z, dtype=np.float64) + k_t
    num = q_t @ S
    o = num / (q_t @ z) if normalize else num
    return o, S, z


def decay_scores_first(q, k, v, gamma: float, normalize: bool = False) -> np.ndarray:
    """Unrolled recurrence as one L x L matrix: A = (q k^T) * D with D from
    decay_weights; numerator A v; normalised: divide by the row sums of A."""
    q, k, v = _f64(q, k, v)
    A = (q @ k.T) * decay_weights(q.shape[0], k.shape[0], gamma)
    num = A @ v
    if not normalize:
        return num
    return _divide(num, A.sum(axis=1))


def decay_chunked(q, k, v, C: int, gamma: float, normalize: bool = False):
    """Chunkwise form of the decayed recurrence (C <= 0 is treated as 1).

    Unrolling the recurrence inside a chunk [s, e) of n rows, with P the state
    after row s - 1:  S_{s+i} = gamma^(i+1) P + sum_{j<=i} gamma^(i-j) k_{s+j}^T v_{s+j}.
    So, for local rows i, j of the chunk:
        inter  = gamma^(i+1) q_i P           (denominator: gamma^(i+1) q_i . z)
        intra  = ((q_c k_c^T) * D) v_c       (denominator: row sums of (q_c k_c^T) * D)
        P     <- gamma^n P + k_c^T diag(gamma^(n-1-j)) v_c
        z     <- gamma^n z + sum_j gamma^(n-1-j) k_j
    Returns (out, S_L, z_L)."""
    if C <= 0:
        C = 1
    q, k, v = _f64(q, k, v)
    L, dk = q.shape
    dv = v.shape[1]
    out = np.zeros((L, dv))
    S = np.zeros((dk, dv))
    z = np.zeros(dk)
    for s in range(0, L, C):
        e = min(s + C, L)
        n = e - s
        qc, kc, vc = q[s:e], k[s:e], v[s:e]
        rows = np.arange(n)
        g_in = float(gamma) ** (rows + 1)
        g_out = float(gamma) ** (n - 1 - rows)
        sc = (qc @ kc.T) * decay_weights(n, n, gamma)
        num = g_in[:, None] * (qc @ S) + sc @ vc
        if normalize:
            den = g_in * (qc @ z) + sc.sum(axis=1)
            out[s:e] = _divide(num, den)
        else:
            out[s:e] = num
        S = float(gamma) ** n * S + kc.T @ (g_out[:, None] * vc)
        z = float(gamma) ** n * z + (g_out[:, None] * kc).sum(axis=0)
    return out, S, z


def decay_chunk_states(k, v, C: int, gamma: float):
    """Per-chunk states as they stand at each chunk's end: S_n = sum over the
    chunk's rows j of gamma^(e-1-j) k_j^T v_j, z_n likewise; with the row count
    of each chunk.  Returns (S [N, dk, dv], z [N, dk], lengths [N])."""
    if C <= 0:
        C = 1
    kf, vf = _f64(k, v)
    L, dk = kf.shape
    N = (L + C - 1) // C
    S = np.zeros((N, dk, vf.shape[1]))
    z = np.zeros((N, dk))
    lengths = np.zeros(N, dtype=np.int64)
    for n in range(N):
        s, e = n * C, min((n + 1) * C, L)
        w = float(gamma) ** (e - 1 - np.arange(s, e))
        S[n] = kf[s:e].T @ (w[:, None] * vf[s:e])
        z[n] = (w[:, None] * kf[s:e]).sum(axis=0)
        lengths[n] = e - s
    return S, z, lengths


def decay_exclusive_scan(S_n: np.ndarray, lengths, gamma: float):
    """P_0 = 0, P_n = gamma^(len_{n-1}) P_{n-1} + S_{n-1}: the state after the rows
    before chunk n; also the total after the last chunk (the final state)."""
    Sf = np.asarray(S_n, dtype=np.float64)
    P = np.zeros_like(Sf)
    run = np.zeros(Sf.shape[1:])
    for n in range(Sf.shape[0]):
        P[n] = run
        run = float(gamma) ** int(lengths[n]) * run + Sf[n]
    return P, run


def brute_force_decay(q, k, v, gamma, normalize: bool = False):
    """o_{i,c} = sum_{j<=i} gamma^(i-j) sum_a q_{i,a} k_{j,a} v_{j,c}  [/ the same
    without v], in exact Fractions (gamma given as a Fraction or an exact float)."""
    def exact(x):
        if isinstance(x, (int, np.integer)):
            return Fraction(int(x))
        return Fraction(float(x))

    g = gamma if isinstance(gamma, Fraction) else Fraction(float(gamma))
    L, dk = len(q), len(q[0])
    dv = len(v[0])
    out = []
    for i in range(L):
        row = []
        den = Fraction(0)
        for j in range(i + 1):
            for a in range(dk):
                den += g ** (i - j) * exact(q[i][a]) * exact(k[j][a])
        for c in range(dv):
            acc = Fraction(0)
            for j in range(i + 1):
                s = Fraction(0)
                for a in range(dk):
                    s += exact(q[i][a]) * exact(k[j][a])
                acc += g ** (i - j) * s * exact(v[j][c])
            row.append(acc / den if normalize else acc)
        out.append(row)
    return out


# ---------------------------------------------------------------------------
# Log-linear attention (the slide deck "Log-Linear Attention": Fenwick-tree
# token partition, the hierarchical mask M, the Fenwick tree recurrence, and
# the chunkwise computation).  Query t sees key s <= t at level
#     level(t, s) = 0 if s == t, else floor(log2(t XOR s)) + 1,
# i.e. level l >= 1 holds the 2^(l-1) keys just below t's prefix with bits
# below l-1 cleared, present when bit l-1 of t is set (t = 7: {7}, {6}, {4, 5},
# {0..3}).  With per-token, per-level weights lam[t, l]:
#     y_t = sum_{s <= t} lam[t, level(t, s)] (q_t . k_s) v_s
# (M[t, s] = lam[t, level(t, s)]); lam = 1 everywhere is linear attention.
# The weights are inputs; no normaliser (the slides give none).
# ---------------------------------------------------------------------------
def loglinear_levels(L: int) -> int:
    """Levels a sequence of L tokens uses: 0 .. ceil(log2(L))."""
    return 1 + max(0, int(L - 1).bit_length())


def loglinear_level(t: int, s: int) -> int:
    """Fenwick level of key s <= t for query t."""
    return 0 if s == t else int(t ^ s).bit_length()


def loglinear_scores_first(q, k, v, lam) -> np.ndarray:
    """(q k^T * M) v with M[t, s] = lam[t, level(t, s)] for s <= t, 0 above."""
    q, k, v = _f64(q, k, v)
    lam = np.asarray(lam, dtype=np.float64)
    L = q.shape[0]
    M = np.zeros((L, L))
    for t in range(L):
        for s_ in range(t + 1):
            M[t, s_] = lam[t, loglinear_level(t, s_)]
    return ((q @ k.T) * M) @ v


def loglinear_recurrent(q, k, v, lam, S0=None, t0: int = 0, return_state: bool = False):
    """The Fenwick tree recurrence over level states S^l (sum of k_s^T v_s over
    level l's bucket): at token t, with b = the position of t's lowest set bit,
    the buckets of levels 0..b at t-1 merge into level b+1, levels 1..b empty,
    level 0 takes k_t^T v_t, higher levels stay; then y_t = sum_l lam[t, l] q_t S^l
    (t = 0: only level 0).

    Row i of q, k, v, lam is token t0 + i; S0 (levels x d_k x d_v) is the state
    after token t0 - 1 (zeros when None).  With return_state, also the level
    states after the last token."""
    q, k, v = _f64(q, k, v)
    lam = np.asarray(lam, dtype=np.float64)
    L, dk = q.shape
    dv = v.shape[1]
    n_lev = lam.shape[1]
    S = np.zeros((n_lev, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    out = np.zeros((L, dv))
    for i in range(L):
        t = t0 + i
        if t > 0:
            b = (t & -t).bit_length() - 1
            merged = S[:b + 1].sum(axis=0)
            S[1:b + 1] = 0.0
            S[b + 1] = merged
        S[0] = np.outer(k[i], v[i])
        out[i] = sum(lam[i, l] * (q[i] @ S[l]) for l in range(n_lev))
    return (out, S) if return_state else out


def loglinear_chunked(q, k, v, lam, C: int) -> np.ndarray:
    """Chunkwise log-linear attention with chunks of C = 2^c rows (C <= 0 is 1).

    Inside a chunk (levels 0..c) the masked scores act directly.  Across chunks,
    a key in chunk c' < chunk n sits at level c + floor(log2(n XOR c')) + 1, so
    the earlier chunks group into buckets of 2^(m-1) whole chunks, one per set
    bit m-1 of n: chunks [h - 2^(m-1), h) with h = n with its bits below m-1
    cleared.  Each bucket enters through its summed state:
        out_n = (q_n k_n^T * M_n) v_n + sum_m diag(lam[., c + m]) q_n S_bucket(n, m).
    """
    if C <= 0:
        C = 1
    if C & (C - 1):
        raise ValueError("chunks of a power of two")
    q, k, v = _f64(q, k, v)
    lam = np.asarray(lam, dtype=np.float64)
    L = q.shape[0]
    cb = C.bit_length() - 1
    N = (L + C - 1) // C
    states = [k[n * C:(n + 1) * C].T @ v[n * C:(n + 1) * C] for n in range(N)]
    out = np.zeros((L, v.shape[1]))
    for n in range(N):
        s, e = n * C, min((n + 1) * C, L)
        rows = np.arange(s, e)
        M = np.zeros((e - s, e - s))
        for i, t in enumerate(rows):
            for j in range(i + 1):
                M[i, j] = lam[t, loglinear_level(int(t), int(rows[j]))]
        acc = ((q[s:e] @ k[s:e].T) * M) @ v[s:e]
        m = 1
        while (1 << (m - 1)) <= n:
            if (n >> (m - 1)) & 1:
                h = (n >> (m - 1)) << (m - 1)
                Sb = sum(states[c_] for c_ in range(h - (1 << (m - 1)), h))
                acc = acc + lam[s:e, cb + m][:, None] * (q[s:e] @ Sb)
            m += 1
        out[s:e] = acc
    return out


def brute_force_loglinear(q, k, v, lam):
    """y_{t,c} = sum_{s<=t} lam[t][level(t, s)] sum_a q_{t,a} k_{s,a} v_{s,c}, exact Fractions."""
    def exact(x):
        if isinstance(x, (int, np.integer)):
            return Fraction(int(x))
        return Fraction(float(x))

    L, dk = len(q), len(q[0])
    out = []
    for t in range(L):
        row = []
        for c in range(len(v[0])):
            acc = Fraction(0)
            for s_ in range(t + 1):
                dot = sum((exact(q[t][a]) * exact(k[s_][a]) for a in range(dk)), Fraction(0))
                acc += exact(lam[t][loglinear_level(t, s_)]) * dot * exact(v[s_][c])
            row.append(acc)
        out.append(row)
    return out


# ---------------------------------------------------------------------------
# Exact softmax attention, the reference FAVOR+ approximates (linear-attention
# page: standard attention softmax(Q K^T / sqrt(d_k)) V, and the FAVOR+ kernel
# phi(q).phi(k) whose expectation is exp(q.k), so that phi applied to inputs
# pre-scaled by d_k^(-1/4) estimates the softmax numerator and denominator).
# ---------------------------------------------------------------------------
def softmax_attention(q, k, v, causal: bool = False, scale: Optional[float] = None) -> np.ndarray:
    """softmax(q k^T * scale) v row by row (scale 1/sqrt(d_k) when omitted); causal
    rows see keys j <= i.  The row maximum is subtracted before exp (the ratio is
    unchanged)."""
    q, k, v = _f64(q, k, v)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[1])
    s = (q @ k.T) * scale
    if causal:
        keep = np.arange(k.shape[0])[None, :] <= np.arange(q.shape[0])[:, None]
        s = np.where(keep, s, -np.inf)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    w = w / w.sum(axis=1, keepdims=True)
    return w @ v


def softmax_attention_loops(q, k, v, causal: bool = False, scale: Optional[float] = None):
    """The same by the definition term by term (Python floats, math.exp, no max
    subtraction): o_i = sum_j e^(s_ij) v_j / sum_j e^(s_ij).  Tiny inputs only."""
    import math
    L, dk = len(q), len(q[0])
    if scale is None:
        scale = 1.0 / math.sqrt(dk)
    out = []
    for i in range(L):
        last = i if causal else len(k) - 1
        e = [math.exp(sum(float(q[i][a]) * float(k[j][a]) for a in range(dk)) * scale) for j in range(last + 1)]
        den = sum(e)
        out.append([sum(e[j] * float(v[j][c]) for j in range(last + 1)) / den for c in range(len(v[0]))])
    return out


# ---------------------------------------------------------------------------
# The delta rule and its gated form (page "Kimi K3 と Qwen 3.8 の Attention 機構
# 比較分析", below called the Kimi/Qwen page: section 3.1, its equation (14):
# before writing, look up what the current key already maps to in the state,
# erase that old prediction along the key, then write the new value; section
# 2.4: the gated form is a global decay of the whole state, the directed erase
# and the residual write; section 3.3.5 works the erase through on two keys;
# the chunking page's closing notes name DeltaNet and Gated DeltaNet as the
# successors of the additive state).  With the state S (d_k x d_v) read as
# o = q S, the write strength beta_t and the gate alpha_t per token:
#     S_t = alpha_t (S_{t-1} - beta_t k_t (k_t^T S_{t-1})) + beta_t k_t v_t^T
#         = alpha_t S_{t-1} + k_t u_t^T,   u_t = beta_t (v_t - alpha_t S_{t-1}^T k_t)
#     o_t = q_t^T S_t                      (read after the update)
# beta = 1, alpha = 1 is the page's worked case (old prediction fully erased);
# alpha = 1 is the delta rule without the gate.  No feature map, no
# normaliser (the page gives neither); keys are used as given (the page's
# example takes unit keys).  All forms compute in float64.
# ---------------------------------------------------------------------------
def _gates(alpha, L: int) -> np.ndarray:
    return np.ones(L) if alpha is None else np.asarray(alpha, dtype=np.float64)


def delta_recurrent(q, k, v, beta, alpha=None, S0=None):
    """The recurrence itself, token by token: u_t = beta_t (v_t - alpha_t S_{t-1}^T
    k_t), S_t = alpha_t S_{t-1} + k_t u_t^T, o_t = q_t^T S_t.  Returns (out, S_L);
    S0 continues from a given state (zero when omitted)."""
    q, k, v = _f64(q, k, v)
    L, dk = q.shape
    dv = v.shape[1]
    b = np.asarray(beta, dtype=np.float64)
    a = _gates(alpha, L)
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    out = np.zeros((L, dv))
    for t in range(L):
        old = a[t] * S                       # the decayed state
        u = b[t] * (v[t] - k[t] @ old)       # the new value minus the old prediction at k_t
        S = old + np.outer(k[t], u)          # erase along k_t and write
        out[t] = q[t] @ S
    return out, S


def delta_step(S, q_t, k_t, v_t, beta_t: float, alpha_t: float = 1.0):
    """One decode step of the (gated) delta rule on one state.  Returns (o, S')."""
    old = float(alpha_t) * np.asarray(S, dtype=np.float64)
    u = float(beta_t) * (np.asarray(v_t, dtype=np.float64) - np.asarray(k_t, dtype=np.float64) @ old)
    S = old + np.outer(k_t, u)
    return np.asarray(q_t, dtype=np.float64) @ S, S


def unit_lower_solve(A: np.ndarray, R: np.ndarray) -> np.ndarray:
    """X with (I + A) X = R for a strictly lower-triangular A, by forward
    substitution row by row (exact on integers)."""
    X = np.zeros_like(R, dtype=np.float64)
    for i in range(R.shape[0]):
        X[i] = R[i] - A[i, :i] @ X[:i]
    return X


def delta_chunked(q, k, v, beta, alpha=None, C: int = 64, S0=None):
    """Chunkwise form of the (gated) delta rule, derived from the recurrence
    (C <= 0 is treated as 1).  Inside a chunk [s, e) with P the state before it
    and g_i the product of the gates of its rows 0..i (local indices):
        alpha_i S_{i-1} = g_i P + sum_{j<i} (g_i / g_j) k_j u_j^T,  so
        u_i = beta_i (v_i - g_i P^T k_i - sum_{j<i} (g_i / g_j)(k_i . k_j) u_j),
    i.e. the unit lower-triangular system (I + A) U = diag(beta)(V - diag(g) K P)
    with A[i, j] = beta_i (k_i . k_j) g_i / g_j for j < i.  Then
        O   = diag(g) Q P + (tril(Q K^T) * G) U,     G[i, j] = g_i / g_j
        P  <- g_n P + K^T diag(g_n / g) U            (n rows in the chunk).
    Returns (out, S_L)."""
    if C <= 0:
        C = 1
    q, k, v = _f64(q, k, v)
    L, dk = q.shape
    dv = v.shape[1]
    b = np.asarray(beta, dtype=np.float64)
    a = _gates(alpha, L)
    P = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    out = np.zeros((L, dv))
    for s in range(0, L, C):
        e = min(s + C, L)
        qc, kc, vc, bc = q[s:e], k[s:e], v[s:e], b[s:e]
        g = np.cumprod(a[s:e])
        G = g[:, None] / g[None, :]
        A = np.tril(bc[:, None] * (kc @ kc.T) * G, -1)
        U = unit_lower_solve(A, bc[:, None] * (vc - g[:, None] * (kc @ P)))
        out[s:e] = g[:, None] * (qc @ P) + (tril(qc @ kc.T) * G) @ U
        P = g[-1] * P + kc.T @ ((g[-1] / g)[:, None] * U)
    return out, P


def delta_chunk_transform(k, beta, alpha=None, C: int = 64):
    """Per chunk n the matrix T_n = (I + A_n)^(-1) diag(beta) of delta_chunked
    (rows and columns the chunk's rows; a short last chunk gives a smaller block),
    as the columns of the forward substitution applied to diag(beta).  Returns a
    list of N arrays."""
    if C <= 0:
        C = 1
    k = np.asarray(k, dtype=np.float64)
    L = k.shape[0]
    b = np.asarray(beta, dtype=np.float64)
    a = _gates(alpha, L)
    out = []
    for s in range(0, L, C):
        e = min(s + C, L)
        g = np.cumprod(a[s:e])
        A = np.tril(b[s:e, None] * (k[s:e] @ k[s:e].T) * (g[:, None] / g[None, :]), -1)
        out.append(unit_lower_solve(A, np.diag(b[s:e])))
    return out


def brute_force_delta(q, k, v, beta, alpha=None):
    """The recurrence in exact rational arithmetic (Fractions of the exact binary
    values, or of given Fractions): nested loops over every state element."""
    def exact(x):
        if isinstance(x, Fraction):
            return x
        if isinstance(x, (int, np.integer)):
            return Fraction(int(x))
        return Fraction(float(x))

    L, dk, dv = len(q), len(q[0]), len(v[0])
    S = [[Fraction(0)] * dv for _ in range(dk)]
    out = []
    for t in range(L):
        at = Fraction(1) if alpha is None else exact(alpha[t])
        bt = exact(beta[t])
        kt = [exact(x) for x in k[t]]
        S = [[at * S[i][c] for c in range(dv)] for i in range(dk)]
        pred = [sum((kt[i] * S[i][c] for i in range(dk)), Fraction(0)) for c in range(dv)]
        u = [bt * (exact(v[t][c]) - pred[c]) for c in range(dv)]
        S = [[S[i][c] + kt[i] * u[c] for c in range(dv)] for i in range(dk)]
        out.append([sum((exact(q[t][i]) * S[i][c] for i in range(dk)), Fraction(0)) for c in range(dv)])
    return out, S


# ---------------------------------------------------------------------------
# mapping over heads
# ---------------------------------------------------------------------------
def over_heads(form: Callable, q, k, v, *args, **kwargs):
    """Apply a single-head form to [H, L, d] arrays; stacks each returned array."""
    results = [form(q[h], k[h], v[h], *args, **kwargs) for h in range(q.shape[0])]
    if isinstance(results[0], tuple):
        return tuple(np.stack([r[i] for r in results]) for i in range(len(results[0])))
    return np.stack(results)


def forward(q_raw, k_raw, v, C: int, causal: bool = True, normalize: bool = False,
            fmap: str = "identity", W=None, in_scale: float = 1.0, gamma: float = 1.0):
    """What the forward entry point returns for one head: (out, S_L, z_L).

    phi is applied to q and k, then the chunked form (causal; with the decayed
    recurrence when gamma != 1) or the state-first form (non-causal, C
    ignored) gives the output.
    """
    qp = apply_phi(q_raw, fmap, W, in_scale) if (fmap != "identity" or in_scale != 1.0) else q_raw
    kp = apply_phi(k_raw, fmap, W, in_scale) if (fmap != "identity" or in_scale != 1.0) else k_raw
    if gamma != 1.0:
        if not causal:
            raise ValueError("the decayed recurrence is causal")
        return decay_chunked(qp, kp, v, C, gamma, normalize)
    if causal:
        return chunked(qp, kp, v, C, normalize)
    out = noncausal_state_first(qp, kp, v, normalize)
    S, z = final_state(kp, v)
    return out, S, z
