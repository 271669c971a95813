"""Seeded synthetic inputs for chunkwise causal linear attention.

This module only *draws* inputs. It holds none of the method's arithmetic
(no feature map, no state, no attention product) and is the one piece of
code shared by the CPU oracle and the HIP path's tests and benchmark.

Every tensor is drawn per (batch*head) slice from
``numpy.random.default_rng([workload_id, tensor_id, bh])`` so that a single
head can be regenerated on its own (the oracle checks sampled heads of the
large workloads without materialising the rest).

Floating-point inputs are drawn as float32 standard normals, scaled, and
rounded to bfloat16 with round-to-nearest-even.  The same bf16 values are
handed to the GPU (as raw 16-bit patterns) and to the oracle (widened to
float64, which is exact).

Integer inputs are uniform on {-3, ..., 3} (each value with probability 1/7).

The FAVOR+ projection W is the method's random draw, so it is an input here:
block-orthogonal Gaussian rows scaled by chi(d) norms, following the
construction of orthogonal random features on the page "Linear Attention /
Performerの理論と実装" (section on FAVOR+, subsection on orthogonal random
features, and its create_orthogonal_random_matrix description).  It is
rounded to bf16 so both sides use identical values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Tuple

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_W = 0, 1, 2, 3
TENSOR_DECODE_Q, TENSOR_DECODE_K, TENSOR_DECODE_V = 4, 5, 6


# ---------------------------------------------------------------------------
# bf16 rounding (input quantisation only)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # NaN is never produced by the generators; guard anyway.
    if np.isnan(x).any():
        raise ValueError("NaN in generator output")
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 (exact)."""
    u = bits.astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Tensor:
    """A generated input: raw storage for the GPU plus exact float64/int64 values."""

    bits: np.ndarray  # uint16 bf16 patterns, or int8 values
    exact: np.ndarray  # float64 (bf16-exact) or int64
    dtype: str  # "bf16" or "i8"


def _normal_bf16(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(scale)
    return f32_to_bf16_bits(x)


def _int_uniform(rng: np.random.Generator, shape, lo: int = -3, hi: int = 3) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.int8)


def head_tensor(workload_id: int, tensor_id: int, bh: int, rows: int, cols: int,
                dtype: str, scale: float = 1.0) -> Tensor:
    """One [rows, cols] slice for head index ``bh`` (row-major)."""
    rng = np.random.default_rng([workload_id, tensor_id, bh])
    if dtype == "bf16":
        bits = _normal_bf16(rng, (rows, cols), scale)
        return Tensor(bits, bf16_bits_to_f64(bits), "bf16")
    if dtype == "i8":
        vals = _int_uniform(rng, (rows, cols))
        return Tensor(vals, vals.astype(np.int64), "i8")
    raise ValueError(dtype)


def full_tensor(workload_id: int, tensor_id: int, BH: int, rows: int, cols: int,
                dtype: str, scale: float = 1.0, want_exact: bool = True) -> Tensor:
    """All heads stacked: shape [BH, rows, cols]."""
    store = np.empty((BH, rows, cols), dtype=np.uint16 if dtype == "bf16" else np.int8)
    for bh in range(BH):
        rng = np.random.default_rng([workload_id, tensor_id, bh])
        if dtype == "bf16":
            store[bh] = _normal_bf16(rng, (rows, cols), scale)
        else:
            store[bh] = _int_uniform(rng, (rows, cols))
    exact = None
    if want_exact:
        exact = bf16_bits_to_f64(store) if dtype == "bf16" else store.astype(np.int64)
    return Tensor(store, exact, dtype)


# ---------------------------------------------------------------------------
# FAVOR+ random projection (the method's random draw, passed in as an input)
# ---------------------------------------------------------------------------
def orthogonal_random_features(m: int, d: int, seed) -> Tuple[np.ndarray, np.ndarray]:
    """Block-orthogonal Gaussian projection W of shape [m, d].

    Each block of d rows is a random orthogonal d x d matrix, with row i
    rescaled by the square root of an independent chi-square(d) draw (so the
    row norms follow the chi(d) law of Gaussian vectors).  ceil(m/d) blocks are
    stacked and the first m rows kept.  Returns (bf16 bits, exact float64).

    The orthogonal matrix is the Q factor of a Gaussian matrix with its columns
    multiplied by the signs of R's diagonal.  That normalisation makes Q
    Haar-distributed, so each row direction is uniform on the sphere and
    phi(q).phi(k) stays an unbiased estimate of exp(q.k); a bare Householder Q
    is not Haar and biases the estimate by a few percent.
    """
    rng = np.random.default_rng(seed)
    blocks = []
    for _ in range((m + d - 1) // d):
        g = rng.standard_normal((d, d))
        qmat, rmat = np.linalg.qr(g)
        qmat = qmat * np.sign(np.diag(rmat))[None, :]
        norms = np.sqrt(rng.chisquare(d, size=d))
        blocks.append(norms[:, None] * qmat)
    w = np.vstack(blocks)[:m].astype(np.float32)
    bits = f32_to_bf16_bits(w)
    return bits, bf16_bits_to_f64(bits)


# ---------------------------------------------------------------------------
# The workloads (shapes, distributions, chunk sizes)
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    H: int
    L: int
    d_in: int
    d_v: int
    dtype: str  # "bf16" or "i8"
    fmap: str  # "identity", "elu1", "favor"
    normalize: bool
    chunks: Tuple[int, ...]
    scale: float = 1.0
    m: int = 0  # FAVOR+ feature count (d_k = m when fmap == "favor")
    return_state: bool = False

    @property
    def BH(self) -> int:
        return self.B * self.H

    @property
    def d_k(self) -> int:
        return self.m if self.fmap == "favor" else self.d_in


WORKLOADS: Dict[int, Workload] = {
    1: Workload(1, "int8-exact-L256-d16", 1, 1, 256, 16, 16, "i8", "identity", False,
                (1, 16, 64, 256)),
    2: Workload(2, "elu1-norm-L2048-d64", 4, 8, 2048, 64, 64, "bf16", "elu1", True,
                (64,), scale=1.0 / math.sqrt(64)),
    3: Workload(3, "identity-L8192-d128", 8, 16, 8192, 128, 128, "bf16", "identity", False,
                (32, 64, 128), scale=1.0 / math.sqrt(128)),
    4: Workload(4, "elu1-norm-L65536-d64", 1, 32, 65536, 64, 64, "bf16", "elu1", True,
                (128,), scale=1.0 / math.sqrt(64), return_state=True),
    5: Workload(5, "favor256-norm-L16384-d64", 2, 12, 16384, 64, 64, "bf16", "favor", True,
                (64,), scale=1.0 / math.sqrt(64), m=256, return_state=True),
}

# Decode that follows workload 5: 256 streams x 12 heads continue from the
# forward's final states; stream s starts from batch (s mod 2) of the forward.
DECODE_STREAMS = 256
DECODE_STEPS = 4096
DECODE_POOL = 256  # distinct seeded step inputs; step t uses pool[t mod 256]


def workload_inputs(w: Workload, BH: int = None, L: int = None, want_exact: bool = True):
    """q, k, v Tensors ([BH, L, d]) and, for FAVOR+, W (bits, exact)."""
    BH = w.BH if BH is None else BH
    L = w.L if L is None else L
    q = full_tensor(w.wid, TENSOR_Q, BH, L, w.d_in, w.dtype, w.scale, want_exact)
    k = full_tensor(w.wid, TENSOR_K, BH, L, w.d_in, w.dtype, w.scale, want_exact)
    v = full_tensor(w.wid, TENSOR_V, BH, L, w.d_v, w.dtype, w.scale, want_exact)
    W = orthogonal_random_features(w.m, w.d_in, [w.wid, TENSOR_W]) if w.fmap == "favor" else None
    return q, k, v, W


def head_inputs(w: Workload, bh: int, L: int = None):
    """q, k, v Tensors ([L, d]) of one head, identical to that head's slice of workload_inputs."""
    L = w.L if L is None else L
    return (head_tensor(w.wid, TENSOR_Q, bh, L, w.d_in, w.dtype, w.scale),
            head_tensor(w.wid, TENSOR_K, bh, L, w.d_in, w.dtype, w.scale),
            head_tensor(w.wid, TENSOR_V, bh, L, w.d_v, w.dtype, w.scale))


def decode_pool(w: Workload, n_states: int, pool: int = DECODE_POOL):
    """Seeded step inputs for the decode: q, k [pool, n_states, d_in], v [pool, n_states, d_v]."""
    q = full_tensor(w.wid, TENSOR_DECODE_Q, pool, n_states, w.d_in, "bf16", w.scale)
    k = full_tensor(w.wid, TENSOR_DECODE_K, pool, n_states, w.d_in, "bf16", w.scale)
    v = full_tensor(w.wid, TENSOR_DECODE_V, pool, n_states, w.d_v, "bf16", w.scale)
    return q, k, v


def favor_study_inputs(seed: int = 123, n: int = 128, d: int = 64, scale: float = 0.4):
    """Inputs of the FAVOR+-vs-softmax error study, shaped like the
    linear-attention page's experiment (one head, n = 128, d = 64, entries
    N(0, 1) * 0.4 from numpy's legacy generator seeded 123, drawn Q, K, V in
    that order), rounded to bf16: q, k, v as [1, n, d] Tensors."""
    rs = np.random.RandomState(seed)
    out = []
    for _ in range(3):
        bits = f32_to_bf16_bits((rs.randn(n, d) * scale).astype(np.float32))[None]
        out.append(Tensor(bits, bf16_bits_to_f64(bits), "bf16"))
    return tuple(out)


def loglinear_weights(seed: int, BH: int, L: int, n_levels: int, lo: float = 0.25, hi: float = 1.25) -> np.ndarray:
    """Per-token level weights for log-linear attention, float32 [BH, L, n_levels],
    uniform on [lo, hi) from a seeded generator."""
    rng = np.random.default_rng([seed, 99])
    return rng.uniform(lo, hi, size=(BH, L, n_levels)).astype(np.float32)


def random_case(seed: int, BH: int, L: int, d_in: int, d_v: int, dtype: str,
                scale: float = 1.0):
    """Free-form seeded case for tests: q, k, v of shape [BH, L, d]."""
    q = full_tensor(1000 + seed, TENSOR_Q, BH, L, d_in, dtype, scale)
    k = full_tensor(1000 + seed, TENSOR_K, BH, L, d_in, dtype, scale)
    v = full_tensor(1000 + seed, TENSOR_V, BH, L, d_v, dtype, scale)
    return q, k, v


# ---------------------------------------------------------------------------
# Inputs of the delta rule (the Kimi/Qwen page's erase-then-write update):
# unit keys as in its two-key example, write strengths and gates per token.
# ---------------------------------------------------------------------------
TENSOR_BETA, TENSOR_ALPHA = 7, 8


def unit_rows_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    """Standard normal rows divided by their Euclidean norm (float64), rounded to
    bf16: unit vectors up to the bf16 rounding of each entry."""
    x = rng.standard_normal(size=shape)
    x = x / np.linalg.norm(x, axis=-1, keepdims=True)
    return f32_to_bf16_bits(x.astype(np.float32))


def delta_inputs(seed: int, BH: int, L: int, d_k: int, d_v: int, gated: bool,
                 beta_lo: float = 0.25, alpha_lo: float = 0.9, want_exact: bool = True):
    """Seeded delta-rule inputs, per (batch*head) slice: q ~ N(0,1)/sqrt(d_k) and
    v ~ N(0,1)/sqrt(d_k) in bf16; unit keys (unit_rows_bf16); write strengths
    beta ~ U(beta_lo, 1) and, when gated, gates alpha ~ U(alpha_lo, 1), float32
    [BH, L].  Returns (q, k, v Tensors, beta, alpha or None)."""
    scale = 1.0 / math.sqrt(d_k)
    q = full_tensor(2000 + seed, TENSOR_Q, BH, L, d_k, "bf16", scale, want_exact)
    v = full_tensor(2000 + seed, TENSOR_V, BH, L, d_v, "bf16", scale, want_exact)
    kb = np.empty((BH, L, d_k), dtype=np.uint16)
    beta = np.empty((BH, L), dtype=np.float32)
    alpha = np.empty((BH, L), dtype=np.float32) if gated else None
    for bh in range(BH):
        kb[bh] = unit_rows_bf16(np.random.default_rng([2000 + seed, TENSOR_K, bh]), (L, d_k))
        beta[bh] = np.random.default_rng([2000 + seed, TENSOR_BETA, bh]).uniform(beta_lo, 1.0, L)
        if gated:
            alpha[bh] = np.random.default_rng([2000 + seed, TENSOR_ALPHA, bh]).uniform(alpha_lo, 1.0, L)
    k = Tensor(kb, bf16_bits_to_f64(kb) if want_exact else None, "bf16")
    return q, k, v, beta, alpha


def delta_head_inputs(seed: int, bh: int, L: int, d_k: int, d_v: int, gated: bool,
                      beta_lo: float = 0.25, alpha_lo: float = 0.9):
    """Head bh of delta_inputs alone: (q, k, v float64 [L, d], beta, alpha or None)."""
    scale = 1.0 / math.sqrt(d_k)
    q = head_tensor(2000 + seed, TENSOR_Q, bh, L, d_k, "bf16", scale).exact
    v = head_tensor(2000 + seed, TENSOR_V, bh, L, d_v, "bf16", scale).exact
    k = bf16_bits_to_f64(unit_rows_bf16(np.random.default_rng([2000 + seed, TENSOR_K, bh]), (L, d_k)))
    beta = np.random.default_rng([2000 + seed, TENSOR_BETA, bh]).uniform(beta_lo, 1.0, L).astype(np.float32)
    alpha = (np.random.default_rng([2000 + seed, TENSOR_ALPHA, bh]).uniform(alpha_lo, 1.0, L).astype(np.float32)
             if gated else None)
    return q, k, v, beta, alpha
