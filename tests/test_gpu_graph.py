"""The library under HIP graph capture: its entry points enqueue kernels only
(no allocation, no memset, no synchronisation), so a captured forward or decode
step replays.  Each test captures once, then replays several times on new
inputs copied into the captured buffers, with eager work and synchronisation
between the replays, and checks every replay bit for bit against the same call
made eagerly on the same inputs (the same kernels: deterministic)."""
import numpy as np
import pytest

import chunked_causal_linear_amd as la
import workloads as wl
from tests.gpu_helpers import dev_bf16, log, torch_cuda

pytestmark = pytest.mark.gpu


def _capture(torch, fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # untimed first call outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _fill(dst, seed):
    q, _, _ = wl.random_case(seed, dst.shape[0], dst.shape[1], dst.shape[2], dst.shape[2], "bf16", 0.125)
    dst.copy_(dev_bf16(q.bits))


def test_graph_grouped_forward_replays():
    """elu+1, normalised, several groups per head: phase 1, the scan and phase 3
    with the workspace, captured as one graph."""
    torch = torch_cuda()
    BH, L, d = 4, 1000, 64
    q, k, v = (torch.empty(BH, L, d, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    for i, t in enumerate((q, k, v)):
        _fill(t, 90 + i)
    f = la.Forward(q, k, v, 64, normalize=True, fmap="elu1", group=3)
    g = _capture(torch, f.run)
    for r in range(3):
        for i, t in enumerate((q, k, v)):
            _fill(t, 100 + 3 * r + i)
        log(f"graph replay {r}: grouped elu+1 forward")
        g.replay()
        torch.cuda.synchronize()
        got = f.o.clone()
        f.run()  # the same call, eagerly
        torch.cuda.synchronize()
        assert torch.equal(got, f.o), r


def test_graph_noalloc_forward_replays():
    """The allocation-free forward (its scratch is the library's own array)."""
    torch = torch_cuda()
    BH, L, d = 2, 1500, 128
    q, k, v = (torch.empty(BH, L, d, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    out = torch.empty(BH, L, d, dtype=torch.bfloat16, device="cuda")
    for i, t in enumerate((q, k, v)):
        _fill(t, 110 + i)
    run = lambda: la.chunked_forward_noalloc(q, k, v, 64, out=out, group=4)  # noqa: E731
    g = _capture(torch, run)
    for r in range(3):
        for i, t in enumerate((q, k, v)):
            _fill(t, 120 + 3 * r + i)
        log(f"graph replay {r}: allocation-free forward")
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        run()
        torch.cuda.synchronize()
        assert torch.equal(got, out), r


def test_graph_decode_steps_replay():
    """A decode step captured once and replayed as consecutive steps: the state
    it updates in place advances by one token per replay, as eager steps do."""
    torch = torch_cuda()
    n, d = 8, 64
    rng = np.random.default_rng([130, 0])
    S0 = torch.from_numpy(rng.standard_normal((n, d, d)).astype(np.float32)).cuda()
    z0 = torch.from_numpy(np.abs(rng.standard_normal((n, d))).astype(np.float32) + 1.0).cuda()
    q, k, v = (torch.empty(n, 1, d, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    S, z = S0.clone(), z0.clone()
    o = torch.empty(n, d, dtype=torch.float32, device="cuda")
    step = lambda: la.recurrent_step(q[:, 0], k[:, 0], v[:, 0], S, z, fmap="elu1", normalize=True, out=o)  # noqa
    g = _capture(torch, step)
    S.copy_(S0)
    z.copy_(z0)
    Se, ze = S0.clone(), z0.clone()
    oe = torch.empty_like(o)
    for r in range(4):
        for i, t in enumerate((q, k, v)):
            _fill(t, 140 + 3 * r + i)
        log(f"graph replay {r}: decode step")
        g.replay()
        torch.cuda.synchronize()
        la.recurrent_step(q[:, 0], k[:, 0], v[:, 0], Se, ze, fmap="elu1", normalize=True, out=oe)
        torch.cuda.synchronize()
        assert torch.equal(o, oe) and torch.equal(S, Se) and torch.equal(z, ze), r
