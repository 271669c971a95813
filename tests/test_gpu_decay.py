"""GPU parity for the decayed recurrence S_t = gamma S_{t-1} + phi(k_t) v_t^T
(linear-attention page, RNN view, where forgetting is introduced), through the
C ABI's _decay entry points, against the oracle's decayed forms.

bf16 band as everywhere: |gpu - oracle| <= 1e-2 * (1 + |oracle|) per element,
the oracle in float64 on the same bf16 values.
"""
import numpy as np
import pytest

import chunked_causal_linear_amd as la
import oracle
import workloads as wl
from tests.gpu_helpers import assert_close, dev_bf16, dev_input, host, log, torch_cuda

pytestmark = pytest.mark.gpu


def _case(seed, BH, L, d_in, d_v, scale=None):
    return wl.random_case(seed, BH, L, d_in, d_v, "bf16", 1.0 / np.sqrt(d_in) if scale is None else scale)


def _oracle(q, k, v, C, normalize, fmap, gamma, W=None, in_scale=1.0):
    outs, Ss, zs = [], [], []
    for h in range(q.shape[0]):
        o, S, z = oracle.forward(q[h], k[h], v[h], C, True, normalize, fmap, W, in_scale, gamma)
        outs.append(o)
        Ss.append(S)
        zs.append(z)
    return np.stack(outs), np.stack(Ss), np.stack(zs)


@pytest.mark.parametrize("C,dk,dv,L,group,norm,fmap,gamma", [
    (64, 128, 128, 700, 0, False, "identity", 0.99), (64, 64, 64, 1000, 3, True, "elu1", 0.95),
    (32, 128, 64, 530, 2, False, "identity", 0.9), (32, 64, 128, 300, 0, True, "elu1", 0.97),
    (128, 128, 128, 900, 0, False, "identity", 0.995), (128, 64, 64, 1300, 2, True, "elu1", 0.9),
    (64, 256, 64, 300, 0, False, "identity", 0.8), (64, 128, 128, 200, 0, False, "identity", 0.5),
    (64, 64, 64, 300, 0, False, "identity", 1.0), (128, 128, 64, 333, 3, True, "elu1", 0.98),
    (32, 256, 32, 200, 2, True, "elu1", 0.93),
    # factored form, the state rescaled at almost every tile; at the edge of
    # its range (TT |log2 gamma| close to 48) for every chunk size
    (64, 128, 128, 700, 0, False, "identity", 0.7), (64, 64, 64, 900, 0, True, "elu1", 0.6),
    (32, 64, 64, 600, 0, False, "identity", 0.6), (128, 64, 64, 900, 0, True, "elu1", 0.78),
    # direct form past that range
    (128, 64, 64, 700, 0, False, "identity", 0.7), (32, 64, 64, 500, 0, True, "elu1", 0.3),
    (64, 256, 64, 300, 0, False, "identity", 0.3), (128, 128, 64, 500, 2, True, "elu1", 0.7)])
def test_decay_forward(C, dk, dv, L, group, norm, fmap, gamma):
    """The forward with a decay: chunks of 32, 64 and 128, several groups (the
    prefixes from decayed phase-1 states and the decayed scan), ragged tails,
    with and without the normaliser, identity and elu+1; gamma = 1 is plain.
    The streaming kernel's two forms of the decay (direct, and factored where
    rows of the tile times |log2 gamma| stay within 48) are both covered."""
    q, k, v = _case(51, 2, L, dk, dv)
    log(f"decay forward C={C} dk={dk} dv={dv} L={L} group={group} norm={norm} fmap={fmap} gamma={gamma}")
    o, S, z = la.chunked_forward(dev_input(q), dev_input(k), dev_input(v), C, normalize=norm, fmap=fmap,
                                 return_state=True, group=group, gamma=gamma)
    ref, refS, refz = _oracle(q.exact, k.exact, v.exact, C, norm, fmap, gamma)
    assert_close(host(o), ref, what="o")
    assert_close(host(S), refS, what="S")
    if norm:
        assert_close(host(z), refz, what="z")


def test_decay_long_groups_and_scale():
    """Few long groups (phase 1 in pieces, each piece's length in the scan's
    decay) and a folded input scale on the identity map."""
    q, k, v = _case(52, 2, 8192, 64, 64)
    for norm, fmap, scale, group in ((True, "elu1", 1.0, 64), (False, "identity", 0.5, 32)):
        log(f"decay long groups norm={norm} fmap={fmap} in_scale={scale} group={group}")
        o, S, z = la.chunked_forward(dev_input(q), dev_input(k), dev_input(v), 64, normalize=norm, fmap=fmap,
                                     in_scale=scale, return_state=True, group=group, gamma=0.999)
        ref, refS, refz = _oracle(q.exact, k.exact, v.exact, 64, norm, fmap, 0.999, None, scale)
        assert_close(host(o), ref, what="o")
        assert_close(host(S), refS, what="S")
        if norm:
            assert_close(host(z), refz, what="z")


def test_decay_favor():
    q, k, v = _case(53, 2, 500, 64, 64, scale=1.0 / 8)
    Wb, W = wl.orthogonal_random_features(64, 64, [53, 3])
    log("decay favor m=64")
    o, S, z = la.chunked_forward(dev_input(q), dev_input(k), dev_input(v), 64, normalize=True, fmap="favor",
                                 W=dev_bf16(Wb), return_state=True, group=2, gamma=0.97)
    ref, refS, refz = _oracle(q.exact, k.exact, v.exact, 64, True, "favor", 0.97, W)
    assert_close(host(o), ref, what="o")
    assert_close(host(S), refS, what="S")
    assert_close(host(z), refz, what="z")


def test_decay_phases():
    """Phase by phase: decayed per-chunk states at each chunk's end, their
    decayed exclusive prefix at group granularity, then phase 3 from it."""
    torch = torch_cuda()
    C, group, gamma = 64, 3, 0.95
    q, k, v = _case(54, 2, 777, 64, 64)
    log("decay phases")
    kd, vd = dev_input(k), dev_input(v)
    S1, _ = la.chunk_states(kd, vd, C, gamma=gamma)
    for h in range(2):
        Sn, _, lens = oracle.decay_chunk_states(k.exact[h], v.exact[h], C, gamma)
        assert_close(host(S1[h]), Sn, what="chunk states")
        P, tot = oracle.decay_exclusive_scan(Sn, lens, gamma)
    S1f, _ = la.state_scan(S1, None, want_final=True, gamma=gamma, L=777, C=C)
    for h in range(2):
        Sn, _, lens = oracle.decay_chunk_states(k.exact[h], v.exact[h], C, gamma)
        P, tot = oracle.decay_exclusive_scan(Sn, lens, gamma)
        assert_close(host(S1[h]), P, what="prefix")
        assert_close(host(S1f[h]), tot, what="total")
    # phase 3 from prefixes at group granularity
    Sg, _ = la.chunk_states(kd, vd, C * group, gamma=gamma)
    la.state_scan(Sg, None, want_final=False, gamma=gamma, L=777, C=C * group)
    o, Sf, _ = la.chunk_output(dev_input(q), kd, vd, C, group, P_prefix=Sg, return_state=True, gamma=gamma)
    ref, refS, _ = _oracle(q.exact, k.exact, v.exact, C, False, "identity", gamma)
    assert_close(host(o), ref, what="o")
    assert_close(host(Sf), refS, what="S")
    torch.cuda.synchronize()


def test_decay_decode_resume():
    """The decayed forward over L1 tokens, then decode steps from its final
    state, matches the decayed recurrence over all tokens."""
    torch = torch_cuda()
    L, L1, d, gamma = 300, 256, 64, 0.97
    q, k, v = _case(55, 3, L, d, d)
    log("decay decode resume")
    qd, kd, vd = dev_input(q), dev_input(k), dev_input(v)
    _, S, z = la.chunked_forward(qd[:, :L1].contiguous(), kd[:, :L1].contiguous(), vd[:, :L1].contiguous(), 64,
                                 normalize=True, fmap="elu1", return_state=True, gamma=gamma)
    outs = []
    for t in range(L1, L):
        o = la.recurrent_step(qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(), S, z,
                              fmap="elu1", normalize=True, gamma=gamma)
        outs.append(host(o))
    got = np.stack(outs, axis=1)
    for h in range(3):
        qp, kp = oracle.phi_elu1(q.exact[h]), oracle.phi_elu1(k.exact[h])
        ref = oracle.decay_state_first(qp, kp, v.exact[h], gamma, True)[0][L1:]
        assert_close(got[h], ref, what=f"decode head {h}")
    torch.cuda.synchronize()


@pytest.mark.parametrize("dk,dv,L,C,gamma,want_z", [
    (64, 64, 1000, 256, 0.99, True), (128, 128, 1300, 320, 0.9, True), (256, 64, 900, 512, 0.999, True),
    (128, 64, 700, 256, 1e-20, True), (64, 128, 2000, 1024, 0.97, False)])
def test_decay_stream_states(dk, dv, L, C, gamma, want_z):
    """Decayed per-run states over runs of 256 rows or more (the streaming
    phase 1: V operands and the ones of z weighted by gamma^(e-1-r)), ragged
    last run, against the oracle's decayed chunk states; gamma = 1e-20 leaves
    each run's last row alone."""
    q, k, v = _case(56, 2, L, dk, dv)
    log(f"decay stream states dk={dk} dv={dv} L={L} C={C} gamma={gamma} want_z={want_z}")
    S, z = la.chunk_states(dev_input(k), dev_input(v), C, gamma=gamma, want_z=want_z)
    for h in range(2):
        Sn, zn, _ = oracle.decay_chunk_states(k.exact[h], v.exact[h], C, gamma)
        assert_close(host(S[h]), Sn, what="states")
        if want_z:
            assert_close(host(z[h]), zn, what="column sums")


@pytest.mark.parametrize("C,dk,dv,L,group,norm,fmap,gamma", [
    (64, 64, 64, 2000, 8, True, "elu1", 0.995), (64, 128, 128, 1500, 4, False, "identity", 0.99),
    (128, 64, 64, 3000, 4, True, "elu1", 0.999), (32, 128, 64, 1200, 8, True, "elu1", 0.98),
    (64, 64, 64, 700, 4, False, "identity", 1e-20), (128, 64, 128, 631, 5, True, "elu1", 0.999)])
def test_decay_forward_stream_phase1(C, dk, dv, L, group, norm, fmap, gamma):
    """Decayed forwards whose groups span 256 rows or more, so that phase 1
    runs on the streaming kernel (elu+1 mapped in it, the weight applied to
    phi(k) in fp32 before its hi/lo split), with every final state; gamma =
    1e-20 runs the direct form."""
    q, k, v = _case(57, 2, L, dk, dv)
    log(f"decay forward stream phase 1 C={C} dk={dk} L={L} group={group} norm={norm} gamma={gamma}")
    o, S, z = la.chunked_forward(dev_input(q), dev_input(k), dev_input(v), C, normalize=norm, fmap=fmap,
                                 return_state=True, group=group, gamma=gamma)
    ref, refS, refz = _oracle(q.exact, k.exact, v.exact, C, norm, fmap, gamma)
    assert_close(host(o), ref, what="o")
    assert_close(host(S), refS, what="S")
    if norm:
        assert_close(host(z), refz, what="z")


def test_decay_favor_stream_phase1():
    """FAVOR+ with the decay in groups of 256 rows (pre-mapped phi(k) with its
    residual: phase 1 on the register-staged kernel, which weights phi(k)
    before it rounds)."""
    q, k, v = _case(58, 2, 1100, 64, 64, scale=1.0 / 8)
    Wb, W = wl.orthogonal_random_features(128, 64, [58, 1])
    log("decay favor stream phase 1 m=128")
    o, S, z = la.chunked_forward(dev_input(q), dev_input(k), dev_input(v), 64, normalize=True, fmap="favor",
                                 W=dev_bf16(Wb), return_state=True, group=4, gamma=0.98)
    ref, refS, refz = _oracle(q.exact, k.exact, v.exact, 64, True, "favor", 0.98, W)
    assert_close(host(o), ref, what="o")
    assert_close(host(S), refS, what="S")
    assert_close(host(z), refz, what="z")
