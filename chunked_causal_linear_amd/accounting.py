"""Algorithmic work and byte counts for chunkwise causal linear attention.

The operation counts follow the chunking page, "attention と線形の間"
(sharin-2a1.pages.dev/parts/chunked.html), section ③ and its Shape type:
per chunk, writing the chunk into the state and reading the state each cost
C*d^2 multiply-accumulates, and building the intra-chunk scores and mixing the
values each cost C^2*d.  Summed over L/C chunks: a fixed part 2*L*d^2 that does
not depend on C and a part 2*L*C*d proportional to C.  The page's counts are
multiply-accumulates; FLOP figures here are 2 x MAC.

``Shape`` keeps the page's square-head closed forms.  ``Work`` generalises
them to d_k != d_v, a ragged last chunk, the normaliser and the feature map, and
adds the byte models used for the roofline.
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Shape:
    """Sequence length L, head width D, chunk size C (square head, d_k = d_v = D)."""

    L: int
    D: int
    C: int

    def state_macs(self) -> int:
        """Writing into and reading from the state: 2 * L * D^2, independent of C."""
        return 2 * self.L * self.D * self.D

    def score_macs(self) -> int:
        """Intra-chunk scores and value mixing: 2 * L * C * D, proportional to C."""
        return 2 * self.L * self.C * self.D

    def macs(self) -> int:
        return self.state_macs() + self.score_macs()

    def intra_memory(self) -> int:
        """Elements of the C x C intra-chunk score block."""
        return self.C * self.C

    def is_full_attention(self) -> bool:
        return self.C >= self.L

    def is_linear(self) -> bool:
        return self.C == 1

    def state_elements(self) -> int:
        """The carried state is D x D whatever L is."""
        return self.D * self.D

    def kv_cache_elements(self) -> int:
        """Keys and values of every token: 2 * L * D."""
        return 2 * self.L * self.D


@dataclasses.dataclass(frozen=True)
class Work:
    """Per-call counts for one forward over BH heads."""

    BH: int
    L: int
    d_in: int
    d_k: int
    d_v: int
    C: int
    normalize: bool = False
    fmap: str = "identity"
    in_bytes: int = 2  # bytes per input element (bf16 = 2, int8 = 1)
    out_bytes: int = 2  # bytes per output element
    state_bytes: int = 4  # fp32 / int32 state

    @property
    def n_chunks(self) -> int:
        C = max(1, self.C)
        return (self.L + C - 1) // C

    def _chunk_sizes(self):
        C = max(1, self.C)
        full, rem = divmod(self.L, C)
        return full, C, rem

    def page_macs(self) -> int:
        """The page's count generalised: state write + read L*d_k*d_v each;
        scores sum over chunks of c^2*d_k, mixing c^2*d_v (full C x C blocks)."""
        full, C, rem = self._chunk_sizes()
        sq = full * C * C + rem * rem
        per_head = 2 * self.L * self.d_k * self.d_v + sq * (self.d_k + self.d_v)
        if self.normalize:
            # denominator: q . z (d_k per token), z update (d_k per token),
            # row sums of the masked block (c^2 per chunk)
            per_head += 2 * self.L * self.d_k + sq
        return self.BH * per_head

    def causal_useful_macs(self) -> int:
        """Only the lower triangle (with diagonal) of each chunk's score block."""
        full, C, rem = self._chunk_sizes()
        tri = full * C * (C + 1) // 2 + rem * (rem + 1) // 2
        per_head = 2 * self.L * self.d_k * self.d_v + tri * (self.d_k + self.d_v)
        if self.normalize:
            per_head += 2 * self.L * self.d_k + tri
        return self.BH * per_head

    def fmap_macs(self) -> int:
        """FAVOR+ projection of q and k: 2 * L * m * d_in per head (elementwise maps: 0)."""
        if self.fmap == "favor":
            return self.BH * 2 * self.L * self.d_k * self.d_in
        return 0

    def page_flops(self) -> int:
        return 2 * (self.page_macs() + self.fmap_macs())

    def fused_bytes(self, return_state: bool = False) -> int:
        """Read q, k (raw width d_in), v once; write o once (+ the final state)."""
        b = self.BH * self.L * ((2 * self.d_in + self.d_v) * self.in_bytes + self.d_v * self.out_bytes)
        if return_state:
            b += self.BH * (self.d_k * self.d_v + (self.d_k if self.normalize else 0)) * self.state_bytes
        return b

    def chunk_state_bytes(self, n: int = None) -> int:
        """Bytes of n per-chunk states (S and, when normalised, z)."""
        n = self.n_chunks if n is None else n
        return self.BH * n * (self.d_k * self.d_v + (self.d_k if self.normalize else 0)) * self.state_bytes


def phase1_bytes(BH: int, L: int, d_k: int, d_v: int, C: int, normalize: bool,
                 in_bytes: int = 2, state_bytes: int = 4) -> int:
    """Read k, v; write one d_k x d_v state (+ d_k normaliser) per chunk."""
    N = (L + max(1, C) - 1) // max(1, C)
    return BH * (L * (d_k + d_v) * in_bytes
                 + N * (d_k * d_v + (d_k if normalize else 0)) * state_bytes)


def scan_bytes(BH: int, N: int, d_k: int, d_v: int, normalize: bool, with_final: bool,
               state_bytes: int = 4) -> int:
    """Read and write every per-chunk state once (+ write the final state)."""
    per = d_k * d_v + (d_k if normalize else 0)
    return BH * per * state_bytes * (2 * N + (1 if with_final else 0))


def decode_bytes(n_states: int, d_in: int, d_k: int, d_v: int, normalize: bool,
                 m_proj: int = 0, in_bytes: int = 2, out_bytes: int = 4) -> int:
    """One decode step: read and write every state (S, z), read q, k, v, write o
    (+ read the FAVOR+ projection once)."""
    state = d_k * d_v + (d_k if normalize else 0)
    return (n_states * (2 * state * 4 + (2 * d_in + d_v) * in_bytes + d_v * out_bytes)
            + m_proj * d_in * in_bytes)
