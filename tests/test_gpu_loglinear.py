"""GPU parity for log-linear attention (slide deck "Log-Linear Attention")
through la_loglinear_forward, against the oracle's chunked log-linear form
(itself pinned to the masked matrix form, the Fenwick recurrence and brute
force).  bf16 band: |gpu - oracle| <= 1e-2 * (1 + |oracle|) per element."""
import numpy as np
import pytest

import chunked_causal_linear_amd as la
import oracle
import workloads as wl
from tests.gpu_helpers import assert_close, dev_bf16, dev_input, host, log, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("BH,L,dk,dv", [(2, 64, 64, 64), (2, 1000, 64, 64), (2, 700, 128, 128),
                                        (1, 4096, 128, 64), (3, 130, 64, 256), (2, 33, 128, 64)])
def test_loglinear_forward(BH, L, dk, dv):
    """One chunk, ragged tails, many Fenwick levels (4096 rows: 64 chunks, bucket
    sums of 1..32 chunks), widths 64..256."""
    torch = torch_cuda()
    q, k, v = wl.random_case(81, BH, L, dk, dv, "bf16", 1.0 / np.sqrt(dk))
    nl = la.loglinear_levels(L)
    assert nl == oracle.loglinear_levels(L)
    lam = wl.loglinear_weights(81, BH, L, nl)
    log(f"loglinear BH={BH} L={L} dk={dk} dv={dv} levels={nl}")
    o = la.loglinear_forward(dev_input(q), dev_input(k), dev_input(v), torch.from_numpy(lam).cuda())
    ref = np.stack([oracle.loglinear_chunked(q.exact[h], k.exact[h], v.exact[h], lam[h].astype(np.float64), 64)
                    for h in range(BH)])
    assert_close(host(o), ref, what="o")


def test_loglinear_unit_weights_is_linear_attention():
    """All level weights 1: the same output as the plain causal forward."""
    torch = torch_cuda()
    q, k, v = wl.random_case(82, 2, 900, 128, 128, "bf16", 1.0 / np.sqrt(128))
    lam = np.ones((2, 900, la.loglinear_levels(900)), dtype=np.float32)
    log("loglinear unit weights")
    o = la.loglinear_forward(dev_input(q), dev_input(k), dev_input(v), torch.from_numpy(lam).cuda())
    ref = np.stack([oracle.chunked(q.exact[h], k.exact[h], v.exact[h], 64)[0] for h in range(2)])
    assert_close(host(o), ref, what="o")


def test_loglinear_benchmarked_shape():
    """The shape the benchmark times: 128 heads x 8192 rows, d = 128, 14 levels
    (128 chunks: bucket sums of 1..64 chunks, the top pyramid level), checked on
    three sampled heads."""
    torch = torch_cuda()
    w = wl.WORKLOADS[3]
    q, k, v, _ = wl.workload_inputs(w, want_exact=False)
    nl = la.loglinear_levels(w.L)
    assert nl == 14
    lam = wl.loglinear_weights(3, w.BH, w.L, nl)
    log(f"loglinear benchmarked shape BH={w.BH} L={w.L} levels={nl}")
    o = host(la.loglinear_forward(dev_bf16(q.bits), dev_bf16(k.bits), dev_bf16(v.bits),
                                  torch.from_numpy(lam).cuda()))
    del q, k, v
    for bh in (0, 77, w.BH - 1):
        qh, kh, vh = wl.head_inputs(w, bh)
        ref = oracle.loglinear_chunked(qh.exact, kh.exact, vh.exact, lam[bh].astype(np.float64), 64)
        worst = assert_close(o[bh], ref, what=f"head {bh}")
        log(f"head {bh} worst ratio {worst:.3f}")


def _step_inputs(seed, n, T, dk, dv, nl):
    q, k, v = wl.random_case(seed, n, T, dk, dv, "bf16", 1.0 / np.sqrt(dk))
    lam = wl.loglinear_weights(seed, n, T, nl)
    return q, k, v, lam


def _run_steps(q, k, v, lam, S, t0, t1, out_dtype):
    """GPU steps at positions t0 .. t1 - 1; row i of q, k, v, lam is position i."""
    torch = torch_cuda()
    outs = []
    for t in range(t0, t1):
        qt, kt, vt = (dev_bf16(np.ascontiguousarray(x.bits[:, t])) for x in (q, k, v))
        lt = torch.from_numpy(np.ascontiguousarray(lam[:, t])).cuda()
        out = torch.empty(qt.shape[0], vt.shape[1], dtype=out_dtype, device="cuda")
        la.recurrent_step_loglinear(qt, kt, vt, lt, S, t, out=out)
        outs.append(host(out))
    return np.stack(outs, axis=1)


@pytest.mark.parametrize("n,T,dk,dv,out", [(3, 300, 64, 64, "f32"), (2, 70, 16, 256, "bf16"),
                                           (2, 130, 128, 32, "f32")])
def test_loglinear_step_from_zero(n, T, dk, dv, out):
    """Steps at positions 0 .. T - 1 from zero level states give the oracle's
    Fenwick tree recurrence, output by output, and its level states at the end
    (merges of up to 9 levels at T = 300)."""
    torch = torch_cuda()
    nl = oracle.loglinear_levels(T)
    q, k, v, lam = _step_inputs(83, n, T, dk, dv, nl)
    log(f"loglinear step from zero n={n} T={T} dk={dk} dv={dv} out={out}")
    S = torch.zeros(n, nl, dk, dv, dtype=torch.float32, device="cuda")
    got = _run_steps(q, k, v, lam, S, 0, T, torch.float32 if out == "f32" else torch.bfloat16)
    Sg = host(S)
    for h in range(n):
        ref, rS = oracle.loglinear_recurrent(q.exact[h], k.exact[h], v.exact[h], lam[h].astype(np.float64),
                                             return_state=True)
        assert_close(got[h], ref, what=f"o stream {h}")
        assert_close(Sg[h], rS, what=f"S stream {h}")


def test_loglinear_step_resume_deep_merge():
    """Steps at positions 1024 .. 1063 from the oracle's level states after
    token 1023 (position 1024 merges eleven levels into level 11), d_k = 128,
    bf16 output, twelve levels kept."""
    torch = torch_cuda()
    n, T0, T1, dk, dv = 2, 1024, 1064, 128, 64
    nl = oracle.loglinear_levels(1100)
    q, k, v, lam = _step_inputs(84, n, T1, dk, dv, nl)
    log(f"loglinear step resume at {T0}, levels={nl}")
    S0, refs, rSs = [], [], []
    for h in range(n):
        lam_h = lam[h].astype(np.float64)
        _, Sa = oracle.loglinear_recurrent(q.exact[h][:T0], k.exact[h][:T0], v.exact[h][:T0], lam_h[:T0],
                                           return_state=True)
        ref, rS = oracle.loglinear_recurrent(q.exact[h][T0:], k.exact[h][T0:], v.exact[h][T0:], lam_h[T0:],
                                             S0=Sa, t0=T0, return_state=True)
        S0.append(Sa)
        refs.append(ref)
        rSs.append(rS)
    S = torch.from_numpy(np.stack(S0).astype(np.float32)).cuda()
    got = _run_steps(q, k, v, lam, S, T0, T1, torch.bfloat16)
    Sg = host(S)
    for h in range(n):
        assert_close(got[h], refs[h], what=f"o stream {h}")
        assert_close(Sg[h], rSs[h], what=f"S stream {h}")


def test_loglinear_steps_match_forward():
    """Decode steps from zero and the chunked forward on the same inputs and
    weights: both against the oracle's masked form, position by position
    (the decode path and the forward path reach the same outputs)."""
    torch = torch_cuda()
    n, T, dk, dv = 2, 200, 64, 128
    nl = la.loglinear_levels(T)
    q, k, v, lam = _step_inputs(85, n, T, dk, dv, nl)
    log("loglinear steps vs forward")
    S = torch.zeros(n, nl, dk, dv, dtype=torch.float32, device="cuda")
    got = _run_steps(q, k, v, lam, S, 0, T, torch.float32)
    fwd = host(la.loglinear_forward(dev_input(q), dev_input(k), dev_input(v), torch.from_numpy(lam).cuda()))
    for h in range(n):
        ref = oracle.loglinear_scores_first(q.exact[h], k.exact[h], v.exact[h], lam[h].astype(np.float64))
        assert_close(got[h], ref, what=f"steps stream {h}")
        assert_close(fwd[h], ref, what=f"forward stream {h}")


def test_loglinear_step_benchmarked_positions():
    """The positions the benchmark's step row and the deepest merge use, at its
    width (d_k = d_v = 128): from the oracle's level states after token 8190,
    steps at 8191 (twelve levels above level 0 hold keys) and 8192 (levels
    0..13 merge into level 14), fifteen levels kept."""
    torch = torch_cuda()
    n, T0, T1, dk, dv = 2, 8191, 8193, 128, 128
    nl = oracle.loglinear_levels(T1)
    assert nl == 15
    q, k, v, lam = _step_inputs(86, n, T1, dk, dv, nl)
    log(f"loglinear step at positions {T0}, {T0 + 1}, levels={nl}")
    S0, refs, rSs = [], [], []
    for h in range(n):
        lam_h = lam[h].astype(np.float64)
        _, Sa = oracle.loglinear_recurrent(q.exact[h][:T0], k.exact[h][:T0], v.exact[h][:T0], lam_h[:T0],
                                           return_state=True)
        ref, rS = oracle.loglinear_recurrent(q.exact[h][T0:], k.exact[h][T0:], v.exact[h][T0:], lam_h[T0:],
                                             S0=Sa, t0=T0, return_state=True)
        S0.append(Sa)
        refs.append(ref)
        rSs.append(rS)
    S = torch.from_numpy(np.stack(S0).astype(np.float32)).cuda()
    got = _run_steps(q, k, v, lam, S, T0, T1, torch.float32)
    Sg = host(S)
    for h in range(n):
        assert_close(got[h], refs[h], what=f"o stream {h}")
        assert_close(Sg[h], rSs[h], what=f"S stream {h}")



@pytest.mark.parametrize("BH,L,dk,dv", [(2, 1, 64, 64), (2, 63, 64, 64), (2, 64, 64, 64), (2, 65, 64, 64),
                                        (2, 1000, 64, 128), (1, 4133, 128, 128), (2, 300, 16, 256)])
def test_loglinear_prefix_levels(BH, L, dk, dv):
    """The level states after a prefix of L tokens (la_loglinear_prefix_levels)
    against the oracle's Fenwick recurrence run over the prefix: one token,
    a chunk and one row either side, buckets of whole chunks (up to 2048 rows at
    L = 4133), one level more than the prefix needs."""
    torch = torch_cuda()
    q, k, v = wl.random_case(87, BH, L, dk, dv, "bf16", 1.0 / np.sqrt(dk))
    nl = oracle.loglinear_levels(L) + 1
    lam = np.ones((L, nl))
    log(f"loglinear prefix levels BH={BH} L={L} dk={dk} dv={dv} levels={nl}")
    S = host(la.loglinear_prefix_levels(dev_input(k), dev_input(v), nl))
    for h in range(BH):
        _, rS = oracle.loglinear_recurrent(q.exact[h], k.exact[h], v.exact[h], lam, return_state=True)
        assert_close(S[h], rS, what=f"levels head {h}")


@pytest.mark.parametrize("BH,L,dk,dv", [(2, 1, 64, 64), (2, 64, 64, 64), (2, 65, 64, 64), (2, 200, 64, 128),
                                        (2, 1000, 128, 256), (1, 4133, 128, 128)])
def test_loglinear_forward_levels(BH, L, dk, dv):
    """The forward's level states after its last token (from its own chunk
    states and bucket pyramid: single nodes of 2 .. 32 chunks at L = 4133)
    against the oracle's Fenwick recurrence over the same tokens, output and
    states, with one level more than the tokens need (written as zero)."""
    torch = torch_cuda()
    q, k, v = wl.random_case(89, BH, L, dk, dv, "bf16", 1.0 / np.sqrt(dk))
    nl = la.loglinear_levels(L)
    lam = wl.loglinear_weights(89, BH, L, nl)
    log(f"loglinear forward levels BH={BH} L={L} dk={dk} dv={dv} levels={nl}+1")
    o, S = la.loglinear_forward(dev_input(q), dev_input(k), dev_input(v), torch.from_numpy(lam).cuda(),
                                return_levels=True, n_state_levels=nl + 1)
    o, S = host(o), host(S)
    assert S.shape == (BH, nl + 1, dk, dv)
    assert not np.any(S[:, nl])
    for h in range(BH):
        lam_h = np.pad(lam[h].astype(np.float64), ((0, 0), (0, 1)))  # the extra level stays empty
        ref, rS = oracle.loglinear_recurrent(q.exact[h], k.exact[h], v.exact[h], lam_h, return_state=True)
        assert_close(o[h], ref, what=f"o head {h}")
        assert_close(S[h], rS, what=f"levels head {h}")


@pytest.mark.parametrize("L,v_shift,oracle_levels", [(16500, 2, True), (262200, 4, False)])
def test_loglinear_long_sequences(L, v_shift, oracle_levels):
    """Sequences long enough for the pyramid's deeper carries (258 chunks: nine
    pyramid levels; 4097 chunks: thirteen): the output against the oracle's
    chunked form, the level states the forward leaves against the oracle's
    recurrence (16,500 tokens) or against la_loglinear_prefix_levels, which sums
    the chunk states in order without the pyramid (262,200 tokens; it is itself
    pinned to the oracle's recurrence).

    Bucket states are sums of up to L/2 outer products and grow as the square
    root of their rows; the products take them as bf16 operands, whose rounding
    grows with them (at unit scale and 16,500 tokens, that rounding alone
    reaches 1.45 of the band at one element: the same figure a CPU model of
    bf16 bucket operands gives).  v is scaled by 2^-v_shift (exact in bf16) so
    that the largest bucket (128 and 2048 chunks) stays below the size of the
    benchmarked shape's (64 chunks at unit scale), where the per-element band
    holds (the model: 0.36 and 0.43 of it); a wrong node would still miss it
    many times over."""
    torch = torch_cuda()
    dk = dv = 64
    q, k, v = wl.random_case(91, 1, L, dk, dv, "bf16", 1.0 / np.sqrt(dk))
    nl = la.loglinear_levels(L)
    lam = wl.loglinear_weights(91, 1, L, nl)
    log(f"loglinear long sequence L={L} levels={nl} v scaled by 2^-{v_shift}")
    scale = 2.0 ** -v_shift
    v_exact = v.exact * scale
    kd, vd = dev_input(k), dev_input(v) * scale
    o, S = la.loglinear_forward(dev_input(q), kd, vd, torch.from_numpy(lam).cuda(), return_levels=True)
    ref = oracle.loglinear_chunked(q.exact[0], k.exact[0], v_exact[0], lam[0].astype(np.float64), 64)
    assert_close(host(o)[0], ref, what="o")
    if oracle_levels:
        _, rS = oracle.loglinear_recurrent(q.exact[0], k.exact[0], v_exact[0], lam[0].astype(np.float64),
                                           return_state=True)
    else:
        rS = host(la.loglinear_prefix_levels(kd, vd))[0].astype(np.float64)
    assert_close(host(S)[0], rS, what="levels")


def test_loglinear_forward_levels_benchmarked_shape():
    """The level states the forward leaves at the benchmarked shape (128 heads x
    8192 rows, d = 128: all fourteen levels hold keys, the top one the
    64-chunk pyramid node), on two sampled heads, against the oracle's
    recurrence."""
    torch = torch_cuda()
    w = wl.WORKLOADS[3]
    q, k, v, _ = wl.workload_inputs(w, want_exact=False)
    nl = la.loglinear_levels(w.L)
    lam = wl.loglinear_weights(3, w.BH, w.L, nl)
    log(f"loglinear forward levels at the benchmarked shape BH={w.BH} L={w.L} levels={nl}")
    _, S = la.loglinear_forward(dev_bf16(q.bits), dev_bf16(k.bits), dev_bf16(v.bits), torch.from_numpy(lam).cuda(),
                                return_levels=True)
    del q, k, v
    for bh in (5, w.BH - 1):
        qh, kh, vh = wl.head_inputs(w, bh)
        _, rS = oracle.loglinear_recurrent(qh.exact, kh.exact, vh.exact, lam[bh].astype(np.float64),
                                           return_state=True)
        worst = assert_close(host(S[bh]), rS, what=f"levels head {bh}")
        log(f"head {bh} worst ratio {worst:.3f}")


@pytest.mark.parametrize("source", ["prefix_levels", "forward"])
def test_loglinear_prefill_then_decode(source):
    """A forward over the first 1500 tokens, the level states at its end (from
    la_loglinear_prefix_levels, or from the forward itself), then decode steps
    at positions 1500 .. 1539: every output against the oracle's masked form
    over the whole sequence."""
    torch = torch_cuda()
    n, T0, T1, dk, dv = 2, 1500, 1540, 128, 64
    nl = oracle.loglinear_levels(T1)
    q, k, v, lam = _step_inputs(88, n, T1, dk, dv, nl)
    log(f"loglinear prefill {T0} ({source}) then decode to {T1}")
    qp, kp, vp = (dev_bf16(np.ascontiguousarray(x.bits[:, :T0])) for x in (q, k, v))
    lam_p = torch.from_numpy(np.ascontiguousarray(lam[:, :T0, :oracle.loglinear_levels(T0)])).cuda()
    if source == "forward":
        o_pre, S = la.loglinear_forward(qp, kp, vp, lam_p, return_levels=True, n_state_levels=nl)
        o_pre = host(o_pre)
    else:
        o_pre = host(la.loglinear_forward(qp, kp, vp, lam_p))
        S = la.loglinear_prefix_levels(kp, vp, nl)
    got = _run_steps(q, k, v, lam, S, T0, T1, torch.float32)
    for h in range(n):
        ref = oracle.loglinear_scores_first(q.exact[h], k.exact[h], v.exact[h], lam[h].astype(np.float64))
        assert_close(o_pre[h], ref[:T0], what=f"prefill head {h}")
        assert_close(got[h], ref[T0:], what=f"decode head {h}")
