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
