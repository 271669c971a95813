"""GPU parity of the streaming phase 1 (runs of whole 64-row tiles at feature
width 64, 128 or 256) against the CPU oracle.

Standalone ``la_chunk_states`` at run lengths of 256 rows and more takes the
streaming kernel with plain K; grouped forwards whose groups are summed in
pieces of that size take it with elu+1 applied in the kernel (split into a
bf16 pair) and with pre-mapped FAVOR+ features and their residual.  Every case
has a ragged last tile, one a last run of a single row.  Tolerance as
everywhere on the bf16 path: |gpu - oracle| <= 1e-2 (1 + |oracle|).
"""
import numpy as np
import pytest

import chunked_causal_linear_amd as la
import oracle
import workloads as wl
from tests.gpu_helpers import assert_close, dev_bf16, dev_input, host, log

pytestmark = pytest.mark.gpu


def _case(seed, BH, L, d_in, d_v, scale=None):
    return wl.random_case(seed, BH, L, d_in, d_v, "bf16", 1.0 / np.sqrt(d_in) if scale is None else scale)


@pytest.mark.parametrize("dk,dv,L,C,want_z", [
    (64, 64, 1000, 256, True), (128, 128, 1300, 320, True), (256, 64, 900, 512, True),
    (64, 128, 2000, 1024, False), (128, 64, 257, 256, True), (256, 32, 700, 256, False),
    (128, 64, 200, 256, True)])
def test_stream_states_plain(dk, dv, L, C, want_z):
    """Per-run states and column sums of plain K over runs of C rows."""
    q, k, v = _case(60, 2, L, dk, dv)
    log(f"stream states dk={dk} dv={dv} L={L} C={C} want_z={want_z}")
    S, z = la.chunk_states(dev_input(k), dev_input(v), C, want_z=want_z)
    ref = [oracle.chunk_states(k.exact[h], v.exact[h], C) for h in range(2)]
    assert_close(host(S), np.stack([r[0] for r in ref]), what="states")
    if want_z:
        assert_close(host(z), np.stack([r[1] for r in ref]), what="column sums")


def _oracle_forward(q, k, v, C, fmap, W=None):
    outs, Ss, zs = [], [], []
    for h in range(q.shape[0]):
        o, S, z = oracle.forward(q[h], k[h], v[h], C, True, True, fmap, W, 1.0)
        outs.append(o)
        Ss.append(S)
        zs.append(z)
    return np.stack(outs), np.stack(Ss), np.stack(zs)


@pytest.mark.parametrize("dk,C,L,group", [(64, 64, 1500, 5), (128, 64, 1111, 4), (256, 64, 1000, 4),
                                          (256, 32, 900, 8)])
def test_stream_states_elu1_forward(dk, C, L, group):
    """Normalised elu+1 forwards in groups of 256 rows or more: phase 1 maps
    phi(k) in the kernel and sums it with its residual."""
    q, k, v = _case(61, 2, L, dk, 64)
    log(f"stream states elu1 forward dk={dk} C={C} L={L} group={group}")
    o, S, z = la.chunked_forward(dev_input(q), dev_input(k), dev_input(v), C, normalize=True, fmap="elu1",
                                 return_state=True, group=group)
    ref, refS, refz = _oracle_forward(q.exact, k.exact, v.exact, C, "elu1")
    assert_close(host(o), ref, what="o")
    assert_close(host(S), refS, what="S")
    assert_close(host(z), refz, what="z")


@pytest.mark.parametrize("m,C,L,group", [(128, 64, 1200, 4), (256, 64, 1000, 5), (64, 128, 1400, 2)])
def test_stream_states_favor_forward(m, C, L, group):
    """FAVOR+ forwards in groups of 256 rows or more: phase 1 reads the
    pre-mapped phi(k) and its residual."""
    q, k, v = _case(62, 2, L, 64, 64, scale=1.0 / 8)
    Wb, W = wl.orthogonal_random_features(m, 64, [62, 1])
    log(f"stream states favor forward m={m} C={C} L={L} group={group}")
    o, S, z = la.chunked_forward(dev_input(q), dev_input(k), dev_input(v), C, normalize=True, fmap="favor",
                                 W=dev_bf16(Wb), return_state=True, group=group)
    ref, refS, refz = _oracle_forward(q.exact, k.exact, v.exact, C, "favor", W)
    assert_close(host(o), ref, what="favor o")
    assert_close(host(S), refS, what="favor S")
    assert_close(host(z), refz, what="favor z")


@pytest.mark.parametrize("C,L,group,scale", [(64, 900, 4, -0.5), (128, 1000, 2, -0.25), (64, 700, 0, -1.0)])
def test_elu1_negative_in_scale(C, L, group, scale):
    """elu+1 of in_scale * x with a negative in_scale: the kernels map
    elu+1(|s| (-x)), flipping the sign bits of the bf16 inputs first (phase 3
    and the streaming phase 1)."""
    q, k, v = _case(63, 2, L, 64, 64)
    log(f"elu1 negative in_scale C={C} L={L} group={group} in_scale={scale}")
    o, S, z = la.chunked_forward(dev_input(q), dev_input(k), dev_input(v), C, normalize=True, fmap="elu1",
                                 in_scale=scale, return_state=True, group=group)
    outs, Ss, zs = [], [], []
    for h in range(2):
        ro, rS, rz = oracle.forward(q.exact[h], k.exact[h], v.exact[h], C, True, True, "elu1", None, scale)
        outs.append(ro)
        Ss.append(rS)
        zs.append(rz)
    assert_close(host(o), np.stack(outs), what="o")
    assert_close(host(S), np.stack(Ss), what="S")
    assert_close(host(z), np.stack(zs), what="z")


@pytest.mark.parametrize("d_in", [16, 32, 64, 128])
@pytest.mark.parametrize("m", [16, 32, 64, 128, 256])
def test_favor_map_every_width(m, d_in):
    """The FAVOR+ map at every feature count (a compile-time parameter of the
    kernel) and input width (16 is padded to 32 inside), over a ragged number
    of rows, fp32 and bf16 outputs, against the oracle's map."""
    torch = __import__("torch")
    rows = 1000 if m <= 64 else 333
    x = wl.random_case(64 + m + d_in, 1, rows, d_in, 16, "bf16", 1.0 / np.sqrt(d_in))[0]
    Wb, W = wl.orthogonal_random_features(m, d_in, [64, m, d_in])
    log(f"favor map m={m} d_in={d_in} rows={rows}")
    ref = oracle.apply_phi(x.exact, "favor", W, 0.7)
    y = la.feature_map(dev_input(x), "favor", W=dev_bf16(Wb), in_scale=0.7, out_dtype=torch.float32)
    assert_close(host(y), ref, tol=1e-4, what="favor fp32")
    yb = la.feature_map(dev_input(x), "favor", W=dev_bf16(Wb), in_scale=0.7)
    assert_close(host(yb), ref, tol=8e-3, what="favor bf16")


def test_scan_large_state_set():
    """The scan of a state set larger than the last-level cache (streamed with
    the non-temporal hint): 64 heads x 128 chunks x 128 x 128 fp32 (537 MB),
    every head's final state and a sample of 64 elements of three heads
    through all chunks, against the oracle's scan of the same values."""
    torch = __import__("torch")
    BH, N, D = 64, 128, 128
    rng = np.random.default_rng(65)
    S_host = rng.standard_normal((BH, N, D, D), dtype=np.float32)
    log(f"scan of a large state set BH={BH} N={N} d={D}x{D}")
    S = torch.from_numpy(S_host).cuda()
    Sf, _ = la.state_scan(S, None)
    cols = rng.choice(D * D, 64, replace=False)
    for h in (0, 31, 63):
        sample = S_host[h].reshape(N, D * D)[:, cols]
        refP, reftot = oracle.exclusive_scan(sample)
        got = host(S[h]).reshape(N, D * D)[:, cols]
        assert_close(got, refP, tol=1e-5, what=f"prefix head {h}")
    refall = np.stack([oracle.exclusive_scan(S_host[h])[1] for h in range(BH)])
    assert_close(host(Sf), refall, tol=1e-5, what="totals")


@pytest.mark.parametrize("d_in,m", [(64, 256), (128, 128), (32, 64)])
def test_decode_favor_input_widths(d_in, m):
    """One FAVOR+ decode step at input widths 32, 64 and 128 (the kernel keeps
    W in LDS sized for d_in <= 64 or <= 128) against the oracle's step."""
    torch = __import__("torch")
    rng = np.random.default_rng([66, d_in, m])
    n, dv = 21, 64
    S0 = rng.standard_normal((n, m, dv)) * 0.5
    z0 = np.abs(rng.standard_normal((n, m))) * 10 + 1
    q, k, v = _case(66 + d_in, 1, n, d_in, dv, scale=0.3)
    Wb, W = wl.orthogonal_random_features(m, d_in, [66, d_in, m])
    S = torch.tensor(S0, dtype=torch.float32, device="cuda")
    z = torch.tensor(z0, dtype=torch.float32, device="cuda")
    s = d_in ** -0.25
    log(f"decode FAVOR+ d_in={d_in} m={m}")
    o = la.recurrent_step(dev_input(q)[0], dev_input(k)[0], dev_input(v)[0], S, z, fmap="favor", W=dev_bf16(Wb),
                          in_scale=s, normalize=True)
    S32, z32 = S0.astype(np.float32).astype(np.float64), z0.astype(np.float32).astype(np.float64)
    for i in range(n):
        qp = oracle.apply_phi(q.exact[0, i][None], "favor", W, s)[0]
        kp = oracle.apply_phi(k.exact[0, i][None], "favor", W, s)[0]
        ro, rS, rz = oracle.recurrent_step(S32[i], z32[i], qp, kp, v.exact[0, i], True)
        assert_close(host(o)[i], ro, tol=1e-4, what="o")
        assert_close(host(S)[i], rS, tol=1e-5, what="S")
        assert_close(host(z)[i], rz, tol=1e-5, what="z")
