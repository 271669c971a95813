"""The allocation-free forward (la_chunked_forward_noalloc) through the C ABI,
against la_chunked_forward with a workspace of its own: two calls in a row, the
second smaller than the first, each needing scratch (phase-1 states of several
groups and their scan).  The two entry points run the same kernels on the same
plan, so their outputs agree bit for bit; one head of each is also checked
against the oracle at the bf16 band."""
import numpy as np
import pytest

import chunked_causal_linear_amd as la
import oracle
import workloads as wl
from chunked_causal_linear_amd import binding as b
from tests.gpu_helpers import assert_close, dev_bf16, dev_input, host, log, torch_cuda

pytestmark = pytest.mark.gpu

SCRATCH = 64 * 1024 * 1024  # LA_NOALLOC_SCRATCH_BYTES in include/la.h

# the first call is the larger one
CASES = [dict(seed=71, BH=4, L=8192, d=64, dv=64, C=128, fmap="elu1", m=0),
         dict(seed=72, BH=2, L=3000, d=64, dv=64, C=64, fmap="favor", m=128)]


def _check_case(c):
    torch = torch_cuda()
    q, k, v = wl.random_case(c["seed"], c["BH"], c["L"], c["d"], c["dv"], "bf16", 1.0 / 8)
    Wb = W = None
    if c["fmap"] == "favor":
        Wb, W = wl.orthogonal_random_features(c["m"], c["d"], [c["seed"], 1])
    qd, kd, vd = dev_input(q), dev_input(k), dev_input(v)
    Wd = dev_bf16(Wb) if Wb is not None else None
    d_k = c["m"] or c["d"]
    ws = la.forward_workspace_bytes(b.LA_BF16, c["BH"], c["L"], c["d"], c["dv"], c["C"], True, True, c["fmap"],
                                    c["m"])
    assert 0 < ws <= SCRATCH, ws
    log(f"noalloc forward BH={c['BH']} L={c['L']} fmap={c['fmap']} C={c['C']} scratch {ws} B")
    ref_o, ref_S, ref_z = la.chunked_forward(qd, kd, vd, c["C"], normalize=True, fmap=c["fmap"], W=Wd,
                                             return_state=True)
    o = torch.empty_like(ref_o)
    S = torch.empty_like(ref_S)
    z = torch.empty_like(ref_z)
    la.chunked_forward_noalloc(qd, kd, vd, c["C"], normalize=True, fmap=c["fmap"], W=Wd, out=o, S_final=S,
                               z_final=z)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(S, ref_S) and torch.equal(z, ref_z)
    h = c["BH"] - 1
    ro, rS, rz = oracle.forward(q.exact[h], k.exact[h], v.exact[h], c["C"], True, True, c["fmap"], W)
    assert_close(host(o)[h], ro, what="o")
    assert_close(host(S)[h], rS, what="S")
    assert_close(host(z)[h], rz, what="z")


def test_noalloc_two_calls_second_smaller():
    for c in CASES:
        _check_case(c)


def test_noalloc_full_favor_workload():
    """Workload 5 at full size with a bf16 output: FAVOR+ mapped inside the kernels
    needs only the phase-1 states (about 16 MB), so the allocation-free forward
    takes it, and agrees bit for bit with the forward given a workspace."""
    torch = torch_cuda()
    w = wl.WORKLOADS[5]
    q, k, v, W = wl.workload_inputs(w, want_exact=False)
    qd, kd, vd, Wd = dev_bf16(q.bits), dev_bf16(k.bits), dev_bf16(v.bits), dev_bf16(W[0])
    del q, k, v
    log(f"noalloc forward at workload 5's full size BH={w.BH} L={w.L}")
    ref_o, ref_S, ref_z = la.chunked_forward(qd, kd, vd, 64, normalize=True, fmap="favor", W=Wd, return_state=True)
    o = torch.empty_like(ref_o)
    S = torch.empty_like(ref_S)
    z = torch.empty_like(ref_z)
    la.chunked_forward_noalloc(qd, kd, vd, 64, normalize=True, fmap="favor", W=Wd, out=o, S_final=S, z_final=z)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(S, ref_S) and torch.equal(z, ref_z)


def test_noalloc_rejects_more_than_its_scratch():
    """A forward whose scratch exceeds the static array is refused before any
    launch: workload 5 with an fp32 output maps q and k beforehand, three
    [24, 16384, 256] bf16 copies."""
    w = wl.WORKLOADS[5]
    ws = la.forward_workspace_bytes(b.LA_BF16, w.BH, w.L, w.d_in, w.d_v, 64, True, True, "favor", w.m)
    assert ws > SCRATCH
    lib = la.lib()
    fake = 0x1000  # never dereferenced: the call fails its size check first
    st = lib.la_chunked_forward_noalloc(fake, fake, fake, b.LA_BF16, w.BH, w.L, w.d_in, w.d_v, 64, 1, 1, 2, fake,
                                        w.m, 1.0, fake, b.LA_F32, None, None, 0, None)
    assert st == b.LA_ERR_UNSUPPORTED
    assert b"scratch" in lib.la_last_error()
