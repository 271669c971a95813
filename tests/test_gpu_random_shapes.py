"""GPU parity over seeded random shapes: head count, ragged lengths, feature and
value widths, chunk sizes, group sizes, feature maps and the normaliser drawn
from a fixed seed, each case against the CPU oracle (bf16 band
|gpu - oracle| <= 1e-2 (1 + |oracle|)).  The draws cover combinations that the
hand-picked cases do not (kernel and phase-1 choices follow from them).

A positive feature map without the normaliser gives outputs that are sums of
~L d-sized terms of both signs (the values), most of which cancel; there the
band gains a part relative to the sum of the terms' magnitudes, which for
positive features is the same forward over |v| (the oracle computes it).  Each
term carries three bf16 roundings of relative size <= 2^-8 (phi(q), phi(k),
and the score or state operand), so the band is
1e-2 (1 + |oracle|) + 3 * 2^-8 (that sum)."""
import numpy as np
import pytest

import chunked_causal_linear_amd as la
import oracle
import workloads as wl
from tests.gpu_helpers import assert_close, assert_close_scaled, dev_bf16, dev_input, host, log

pytestmark = pytest.mark.gpu


def _draw(i):
    r = np.random.default_rng([77, i])
    fmap = ["identity", "elu1", "favor"][int(r.integers(0, 3))]
    d_in = int(r.choice([64, 128])) if fmap != "favor" else 64
    m = int(r.choice([64, 128, 256])) if fmap == "favor" else 0
    d_k = m if fmap == "favor" else d_in
    C = int(r.choice([32, 64, 128]))
    if d_k == 256 and C == 128:
        C = 64
    d_v = int(r.choice([32, 64, 128])) if d_k != 256 else int(r.choice([32, 64]))
    L = int(r.integers(1, 1400))
    BH = int(r.integers(1, 4))
    normalize = fmap != "identity" and bool(r.integers(0, 2)) or fmap == "favor"
    group = int(r.choice([0, 0, 1, 2, 3, 5]))
    return dict(fmap=fmap, d_in=d_in, m=m, C=C, d_v=d_v, L=L, BH=BH, normalize=normalize, group=group)


@pytest.mark.parametrize("i", range(40))
def test_random_shape(i):
    c = _draw(i)
    log(f"random shape {i}: {c}")
    q, k, v = wl.random_case(78 + i, c["BH"], c["L"], c["d_in"], c["d_v"], "bf16",
                             (1.0 / 8) if c["fmap"] == "favor" else 1.0 / np.sqrt(c["d_in"]))
    W = Wb = None
    if c["fmap"] == "favor":
        Wb, W = wl.orthogonal_random_features(c["m"], c["d_in"], [78, i])
    o, S, z = la.chunked_forward(dev_input(q), dev_input(k), dev_input(v), c["C"], normalize=c["normalize"],
                                 fmap=c["fmap"], W=dev_bf16(Wb) if Wb is not None else None, return_state=True,
                                 group=c["group"])
    cancelling = c["fmap"] != "identity" and not c["normalize"]
    for h in range(c["BH"]):
        ro, rS, rz = oracle.forward(q.exact[h], k.exact[h], v.exact[h], c["C"], True, c["normalize"], c["fmap"],
                                    W, 1.0)
        if cancelling:
            mag, _, _ = oracle.forward(q.exact[h], k.exact[h], np.abs(v.exact[h]), c["C"], True, False, c["fmap"],
                                       W, 1.0)
            assert_close_scaled(host(o)[h], ro, mag, 3 * 2.0 ** -8, what=f"o head {h}")
        else:
            assert_close(host(o)[h], ro, what=f"o head {h}")
        assert_close(host(S)[h], rS, what=f"S head {h}")
        if c["normalize"]:
            assert_close(host(z)[h], rz, what=f"z head {h}")


def _draw_decay(i):
    r = np.random.default_rng([79, i])
    fmap = ["identity", "elu1"][int(r.integers(0, 2))]
    d_k = int(r.choice([64, 128]))
    C = int(r.choice([32, 64, 128]))
    d_v = int(r.choice([64, 128]))
    L = int(r.integers(1, 1400))
    BH = int(r.integers(1, 3))
    normalize = fmap == "elu1" and bool(r.integers(0, 2))
    group = int(r.choice([0, 0, 1, 2, 5]))
    gamma = float(r.choice([0.9, 0.99, 0.999]))
    return dict(fmap=fmap, d_k=d_k, C=C, d_v=d_v, L=L, BH=BH, normalize=normalize, group=group, gamma=gamma)


@pytest.mark.parametrize("i", range(20))
def test_random_shape_decay(i):
    """The decayed recurrence (gamma < 1) over seeded random streaming shapes."""
    c = _draw_decay(i)
    log(f"random decayed shape {i}: {c}")
    q, k, v = wl.random_case(80 + i, c["BH"], c["L"], c["d_k"], c["d_v"], "bf16", 1.0 / np.sqrt(c["d_k"]))
    o, S, z = la.chunked_forward(dev_input(q), dev_input(k), dev_input(v), c["C"], normalize=c["normalize"],
                                 fmap=c["fmap"], return_state=True, group=c["group"], gamma=c["gamma"])
    cancelling = c["fmap"] != "identity" and not c["normalize"]
    for h in range(c["BH"]):
        ro, rS, rz = oracle.forward(q.exact[h], k.exact[h], v.exact[h], c["C"], True, c["normalize"], c["fmap"],
                                    None, 1.0, c["gamma"])
        if cancelling:
            mag, _, _ = oracle.forward(q.exact[h], k.exact[h], np.abs(v.exact[h]), c["C"], True, False, c["fmap"],
                                       None, 1.0, c["gamma"])
            assert_close_scaled(host(o)[h], ro, mag, 3 * 2.0 ** -8, what=f"o head {h}")
        else:
            assert_close(host(o)[h], ro, what=f"o head {h}")
        assert_close(host(S)[h], rS, what=f"S head {h}")
        if c["normalize"]:
            assert_close(host(z)[h], rz, what=f"z head {h}")


@pytest.mark.parametrize("i", range(12))
def test_random_shape_loglinear(i):
    """Log-linear attention over seeded random lengths (odd chunk counts and
    ragged tails exercise the pyramid's groups of eight and its tail) and
    widths."""
    torch = __import__("torch")
    r = np.random.default_rng([83, i])
    BH, L = int(r.integers(1, 3)), int(r.integers(65, 3000))
    dk, dv = int(r.choice([64, 128])), int(r.choice([64, 128, 256]))
    q, k, v = wl.random_case(84 + i, BH, L, dk, dv, "bf16", 1.0 / np.sqrt(dk))
    nl = la.loglinear_levels(L)
    lam = wl.loglinear_weights(84 + i, BH, L, nl)
    log(f"random loglinear {i}: BH={BH} L={L} dk={dk} dv={dv} levels={nl}")
    o = la.loglinear_forward(dev_input(q), dev_input(k), dev_input(v), torch.from_numpy(lam).cuda())
    ref = np.stack([oracle.loglinear_chunked(q.exact[h], k.exact[h], v.exact[h], lam[h].astype(np.float64), 64)
                    for h in range(BH)])
    assert_close(host(o), ref, what="o")


@pytest.mark.parametrize("i", range(12))
def test_random_three_phases(i):
    """la_chunk_states at group granularity (runs of C * group rows: the
    streaming or the register-staged kernel by size), la_state_scan and
    la_chunk_output against the oracle's forward, over seeded random shapes."""
    r = np.random.default_rng([85, i])
    BH, L = int(r.integers(1, 3)), int(r.integers(1, 2500))
    d_k, d_v = int(r.choice([64, 128])), int(r.choice([64, 128]))
    C = int(r.choice([32, 64, 128]))
    group = int(r.choice([1, 2, 4, 8]))
    q, k, v = wl.random_case(86 + i, BH, L, d_k, d_v, "bf16", 1.0 / np.sqrt(d_k))
    log(f"random three phases {i}: BH={BH} L={L} d_k={d_k} d_v={d_v} C={C} group={group}")
    qd, kd, vd = dev_input(q), dev_input(k), dev_input(v)
    S, _ = la.chunk_states(kd, vd, C * group)
    la.state_scan(S, None, want_final=False)
    o, Sf, _ = la.chunk_output(qd, kd, vd, C, group, P_prefix=S, return_state=True)
    for h in range(BH):
        ro, rS, _ = oracle.forward(q.exact[h], k.exact[h], v.exact[h], C)
        assert_close(host(o)[h], ro, what=f"o head {h}")
        assert_close(host(Sf)[h], rS, what=f"S head {h}")
