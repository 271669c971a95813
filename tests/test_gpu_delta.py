"""GPU parity for the delta rule and its gated form (page "Kimi K3 と Qwen 3.8 の
Attention 機構比較分析", section 3.1 equation (14) and section 2.4) through the
C ABI: the per-chunk transform, the chunked forward and the decode step,
against the oracle's chunked form and decode step (themselves pinned to the
recurrence, exact brute force and the page's two-key example).

bf16 band: |gpu - oracle| <= 1e-2 (1 + |oracle|) per element; the decode step
(fp32 state and arithmetic) at 1e-4.  Inputs: unit keys, q and v drawn
N(0,1)/sqrt(d_k), write strengths U(0.25, 1), gates U(0.9, 1)
(workloads.delta_inputs)."""
import numpy as np
import pytest

import chunked_causal_linear_amd as la
import oracle
import workloads as wl
from tests.gpu_helpers import assert_close, dev_bf16, host, log, torch_cuda

pytestmark = pytest.mark.gpu


def _perm_pos(j: int) -> int:
    """Stored position of column j in a row of T (include/la.h, la_delta_chunk_transform)."""
    jj = j % 32
    return (j // 32) * 32 + (8 * (jj // 4) + jj % 4 if jj < 16 else 8 * ((jj - 16) // 4) + 4 + jj % 4)


PERM = np.array([_perm_pos(j) for j in range(64)])


def _dev_f32(a):
    torch = torch_cuda()
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _case(seed, BH, L, dk, dv, gated):
    q, k, v, beta, alpha = wl.delta_inputs(seed, BH, L, dk, dv, gated)
    return q, k, v, beta, alpha


def _oracle(q, k, v, beta, alpha, h):
    a = None if alpha is None else alpha[h].astype(np.float64)
    return oracle.delta_chunked(q.exact[h], k.exact[h], v.exact[h], beta[h].astype(np.float64), a, 64)


def test_permutation_is_a_bijection():
    assert sorted(PERM.tolist()) == list(range(64))


@pytest.mark.parametrize("BH,L,dk,gated", [(2, 64, 64, False), (2, 200, 128, True), (3, 130, 64, True),
                                           (1, 1, 128, False), (2, 65, 128, True)])
def test_delta_transform(BH, L, dk, gated):
    """T = (I + A)^-1 diag(beta) per chunk of 64 rows and the gates' log2 products."""
    q, k, v, beta, alpha = _case(1, BH, L, dk, 64, gated)
    log(f"delta transform BH={BH} L={L} dk={dk} gated={gated}")
    T, lg = la.delta_chunk_transform(dev_bf16(k.bits), _dev_f32(beta), _dev_f32(alpha))
    T, lg = host(T), host(lg)
    N = (L + 63) // 64
    assert T.shape == (BH, N, 64, 64) and lg.shape == (BH, N, 64)
    for h in range(BH):
        a = None if alpha is None else alpha[h].astype(np.float64)
        refs = oracle.delta_chunk_transform(k.exact[h], beta[h].astype(np.float64), a, 64)
        assert len(refs) == N
        for n, ref in enumerate(refs):
            m = ref.shape[0]
            got = T[h, n][:, PERM]  # back to natural column order
            assert_close(got[:m, :m], ref, what=f"T head {h} chunk {n}")
            assert np.all(got[:m, m:] == 0), "columns past the end carry a zero strength"
            g = np.ones(m) if a is None else a[n * 64:n * 64 + m]
            assert_close(lg[h, n, :m], np.log2(np.cumprod(g)), tol=1e-4, what=f"lg head {h} chunk {n}")


@pytest.mark.parametrize("BH,L,dk,dv,gated", [(2, 64, 64, 64, False), (2, 333, 128, 64, True),
                                              (1, 1000, 128, 128, False), (3, 200, 64, 256, True),
                                              (2, 65, 64, 64, True), (1, 1, 128, 64, False),
                                              (2, 700, 128, 128, True), (4, 129, 64, 128, False)])
def test_delta_forward(BH, L, dk, dv, gated):
    """The chunked forward and its final state: one chunk, ragged tails (a last
    chunk of one row), one and several value tiles, with and without gates."""
    q, k, v, beta, alpha = _case(2, BH, L, dk, dv, gated)
    log(f"delta forward BH={BH} L={L} dk={dk} dv={dv} gated={gated}")
    o, S = la.delta_forward(dev_bf16(q.bits), dev_bf16(k.bits), dev_bf16(v.bits), _dev_f32(beta), _dev_f32(alpha),
                            return_state=True)
    o, S = host(o), host(S)
    for h in range(BH):
        ref, refS = _oracle(q, k, v, beta, alpha, h)
        worst = assert_close(o[h], ref, what=f"o head {h}")
        assert_close(S[h], refS, what=f"S head {h}")
        log(f"head {h} worst ratio {worst:.3f}")


def test_delta_forward_full_strength_orthogonal_keys_is_linear_attention():
    """Keys orthogonal to every earlier key and beta = 1: the erase finds nothing,
    so the output is causal linear attention (the oracle's plain chunked form)."""
    torch = torch_cuda()
    BH, L, d = 2, 128, 128
    rng = np.random.default_rng([9, 9])
    kk = np.stack([np.eye(d)[rng.permutation(d)] * rng.choice([-1.0, 1.0], (L, 1)) for _ in range(BH)])
    kb = wl.f32_to_bf16_bits(kk.astype(np.float32))
    q, _, v, _, _ = _case(3, BH, L, d, d, False)
    beta = np.ones((BH, L), dtype=np.float32)
    log("delta forward, orthogonal keys, full strength")
    o = host(la.delta_forward(dev_bf16(q.bits), dev_bf16(kb), dev_bf16(v.bits), _dev_f32(beta)))
    for h in range(BH):
        ref = oracle.chunked(q.exact[h], kk[h], v.exact[h], 64)[0]
        assert_close(o[h], ref, what=f"head {h}")
    del torch


@pytest.mark.parametrize("n,dk,dv,gated,out", [(64, 64, 64, True, "f32"), (300, 128, 128, False, "f32"),
                                               (33, 256, 64, True, "bf16"), (17, 16, 256, True, "f32"),
                                               (40, 256, 256, False, "f32"), (5, 32, 16, True, "f32")])
def test_delta_decode_step(n, dk, dv, gated, out):
    """One decode step from random fp32 states, checked with fp32 arithmetic."""
    torch = torch_cuda()
    q, k, v, beta, alpha = _case(4, 1, n, dk, dv, gated)
    rng = np.random.default_rng([4, 5])
    S0 = (rng.standard_normal((n, dk, dv)) * 0.1).astype(np.float32)
    Sd = torch.from_numpy(S0.copy()).cuda()
    log(f"delta decode n={n} dk={dk} dv={dv} gated={gated} out={out}")
    o = torch.empty(n, dv, dtype=torch.float32 if out == "f32" else torch.bfloat16, device="cuda")
    la.recurrent_step_delta(dev_bf16(q.bits[0]), dev_bf16(k.bits[0]), dev_bf16(v.bits[0]), Sd, _dev_f32(beta[0]),
                            _dev_f32(None if alpha is None else alpha[0]), out=o)
    o, Sh = host(o), host(Sd)
    tol = 1e-4 if out == "f32" else 1e-2
    for i in range(n):
        a = 1.0 if alpha is None else float(alpha[0, i])
        ro, rS = oracle.delta_step(S0[i].astype(np.float64), q.exact[0, i], k.exact[0, i], v.exact[0, i],
                                   float(beta[0, i]), a)
        assert_close(o[i], ro, tol=tol, what=f"o state {i}")
        assert_close(Sh[i], rS, tol=1e-4, what=f"S state {i}")


def test_delta_forward_then_decode_resumes():
    """Forward over the first L1 tokens, then decode steps from its final state,
    gives the forward over all L tokens (the recurrence's resume)."""
    torch = torch_cuda()
    BH, L, L1, dk, dv = 3, 300, 257, 128, 64
    q, k, v, beta, alpha = _case(5, BH, L, dk, dv, True)
    log("delta forward then decode")
    qd, kd, vd = dev_bf16(q.bits), dev_bf16(k.bits), dev_bf16(v.bits)
    bd, ad = _dev_f32(beta), _dev_f32(alpha)
    _, S = la.delta_forward(qd[:, :L1].contiguous(), kd[:, :L1].contiguous(), vd[:, :L1].contiguous(),
                            bd[:, :L1].contiguous(), ad[:, :L1].contiguous(), return_state=True)
    ref = [_oracle(q, k, v, beta, alpha, h)[0] for h in range(BH)]
    for t in range(L1, L):
        o = host(la.recurrent_step_delta(qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(), S,
                                         bd[:, t].contiguous(), ad[:, t].contiguous()))
        for h in range(BH):
            assert_close(o[h], ref[h][t], what=f"step {t} head {h}")
    del torch


def test_delta_headline_shape_sampled_heads():
    """128 heads x 8192 rows, d = 128 (the shape the benchmark times), gated:
    three sampled heads against the oracle, outputs and final states."""
    w = wl.WORKLOADS[3]
    q, k, v, beta, alpha = wl.delta_inputs(3, w.BH, w.L, w.d_k, w.d_v, True, want_exact=False)
    log(f"delta forward at BH={w.BH} L={w.L} d={w.d_k}")
    o, S = la.delta_forward(dev_bf16(q.bits), dev_bf16(k.bits), dev_bf16(v.bits), _dev_f32(beta), _dev_f32(alpha),
                            return_state=True)
    o, S = host(o), host(S)
    del q, k, v
    for bh in (0, 77, w.BH - 1):
        qh, kh, vh, bh_, ah = wl.delta_head_inputs(3, bh, w.L, w.d_k, w.d_v, True)
        ref, refS = oracle.delta_chunked(qh, kh, vh, bh_.astype(np.float64), ah.astype(np.float64), 64)
        worst = assert_close(o[bh], ref, what=f"o head {bh}")
        assert_close(S[bh], refS, what=f"S head {bh}")
        log(f"head {bh} worst ratio {worst:.3f}")
