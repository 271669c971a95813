"""GPU parity of FAVOR+ mapped inside the streaming kernels (page "Linear
Attention / Performerの理論と実装", the positive random features and the
normalised causal form): 64 input features, m in {64, 128, 256} random
features, chunks of 64, bf16 outputs.  The kernels map q and k from the raw
tiles with W held in LDS; the oracle maps in float64 from the same bf16 inputs
and W.

Band: |gpu - oracle| <= 1e-2 (1 + |oracle|) per element, outputs, final
states and normalisers.  Cases: ragged lengths (one row, one chunk plus a
row), one and several groups, phase-1 runs finer than the groups, several
value tiles, with and without the normaliser and the final state, an input
scale other than the workload's."""

import numpy as np
import pytest

import chunked_causal_linear_amd as la
import oracle
import workloads as wl
from chunked_causal_linear_amd import binding as b
from tests.gpu_helpers import assert_close, dev_bf16, dev_input, host, log, torch_cuda

pytestmark = pytest.mark.gpu


def _oracle(q, k, v, normalize, W, in_scale):
    outs, Ss, zs = [], [], []
    for h in range(q.shape[0]):
        o, S, z = oracle.forward(q[h], k[h], v[h], 64, True, normalize, "favor", W, in_scale)
        outs.append(o)
        Ss.append(S)
        zs.append(z)
    return np.stack(outs), np.stack(Ss), np.stack(zs)


CASES = [
    # m, BH, L, group, d_v, normalize, return_state, in_scale
    (64, 2, 700, 0, 64, True, True, 1.0),
    (64, 3, 65, 1, 128, False, True, 1.0),
    (64, 2, 4096, 32, 64, True, True, 1.0),  # phase-1 runs of 512 rows (four per group)
    (128, 2, 1000, 3, 64, True, True, 1.0),
    (128, 1, 1, 0, 64, True, True, 1.0),
    (128, 2, 333, 0, 256, True, True, 0.7),
    (256, 2, 600, 2, 64, True, True, 1.0),
    (256, 2, 1000, 0, 256, True, False, 1.0),
    (256, 3, 130, 1, 64, True, False, 1.6),
    # Without the normaliser the output sums terms of both signs, up to ~70x
    # larger than the result at scale 1.6, where bf16 operands alone (phi(q),
    # the packed state, the scores) exceed the band: scale 1 there.
    (256, 3, 130, 1, 64, False, False, 1.0),
    (256, 2, 2048, 16, 128, True, True, 1.0),  # runs of 512 rows (two per group)
]


@pytest.mark.parametrize("m,BH,L,group,dv,norm,state,s", CASES)
def test_favor_fused(m, BH, L, group, dv, norm, state, s):
    q, k, v = wl.random_case(31, BH, L, 64, dv, "bf16", 1.0 / 8)
    Wb, W = wl.orthogonal_random_features(m, 64, [31, m])
    log(f"favor fused m={m} BH={BH} L={L} group={group} dv={dv} norm={norm} state={state} s={s}")
    res = la.chunked_forward(dev_input(q), dev_input(k), dev_input(v), 64, normalize=norm, fmap="favor",
                             W=dev_bf16(Wb), in_scale=s, return_state=state, group=group)
    o = res[0] if state else res
    ref, refS, refz = _oracle(q.exact, k.exact, v.exact, norm, W, s)
    worst = assert_close(host(o), ref, what="o")
    if state:
        assert_close(host(res[1]), refS, what="S")
        if norm:
            assert_close(host(res[2]), refz, what="z")
    log(f"worst ratio {worst:.3f}")


def test_favor_fused_is_the_bf16_path():
    """With a bf16 output the forward needs no mapped copies: a workspace too
    small for one copy of phi(k) is enough, while the fp32 output (mapped
    beforehand) asks for more."""
    torch = torch_cuda()
    BH, L, m, dv = 2, 4096, 128, 64
    q, k, v = wl.random_case(32, BH, L, 64, dv, "bf16", 1.0 / 8)
    Wb, W = wl.orthogonal_random_features(m, 64, [32, m])
    qd, kd, vd, Wd = dev_input(q), dev_input(k), dev_input(v), dev_bf16(Wb)
    small = BH * L * m * 2 // 2  # half of one mapped copy; four groups' states take a quarter of it
    ws = torch.empty(small, dtype=torch.uint8, device="cuda")
    lib = b.lib()
    outs = {}
    for name, dt in (("bf16", torch.bfloat16), ("f32", torch.float32)):
        o = torch.empty(BH, L, dv, dtype=dt, device="cuda")
        log(f"favor fused path check, out {name}")
        st = lib.la_chunked_forward(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), b.LA_BF16, BH, L, 64, dv, 64, 1, 1,
                                    b.FMAPS["favor"], Wd.data_ptr(), m, 1.0, o.data_ptr(),
                                    b.LA_BF16 if name == "bf16" else b.LA_F32, None, None, 16, ws.data_ptr(), small,
                                    None)
        outs[name] = (st, o)
    assert outs["bf16"][0] == b.LA_OK, lib.la_last_error()
    assert outs["f32"][0] == b.LA_ERR_WORKSPACE
    ref = _oracle(q.exact, k.exact, v.exact, True, W, 1.0)[0]
    assert_close(host(outs["bf16"][1]), ref, what="o")


def test_favor_fused_matches_premapped_path():
    """The same inputs through the fused kernels (bf16 out) and through the
    mapped-beforehand path (fp32 out): both within the band of the oracle."""
    BH, L, m, dv = 2, 1500, 256, 64
    q, k, v = wl.random_case(33, BH, L, 64, dv, "bf16", 1.0 / 8)
    Wb, W = wl.orthogonal_random_features(m, 64, [33, m])
    torch = torch_cuda()
    log("favor fused against the mapped path")
    args = (dev_input(q), dev_input(k), dev_input(v), 64)
    kw = dict(normalize=True, fmap="favor", W=dev_bf16(Wb), return_state=True)
    o1, S1, z1 = la.chunked_forward(*args, **kw)
    o2, S2, z2 = la.chunked_forward(*args, out_dtype=torch.float32, **kw)
    ref, refS, refz = _oracle(q.exact, k.exact, v.exact, True, W, 1.0)
    for tag, o, S, z in (("fused", o1, S1, z1), ("mapped", o2, S2, z2)):
        assert_close(host(o), ref, what=f"{tag} o")
        assert_close(host(S), refS, what=f"{tag} S")
        assert_close(host(z), refz, what=f"{tag} z")
