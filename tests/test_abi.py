"""The C ABI library on the CPU: it loads, exports every symbol include/la.h
declares, and rejects invalid arguments before launching anything (no GPU
needed; no call here reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import chunked_causal_linear_amd as la
from chunked_causal_linear_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def declared_functions(header=HEADER):
    src = open(header, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_0-9]+)\s*\(", src)))


def test_library_loads_and_exports_header_symbols():
    lib = la.lib()
    names = declared_functions()
    assert "la_chunked_forward" in names and "la_recurrent_step" in names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported
    assert set(b.EXPORTS) == set(names)


def test_probe_library_exports_and_rejects_bad_arguments():
    """libla_probe.so (include/la_probe.h, the matrix-core rate and read
    bandwidth probes) loads and exports what its header declares; invalid
    arguments return -1 unlaunched."""
    path = os.path.join(ROOT, "chunked_causal_linear_amd", "libla_probe.so")
    names = declared_functions(os.path.join(ROOT, "include", "la_probe.h"))
    assert names == ["la_probe_mfma", "la_probe_read"]
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported
    lib = ctypes.CDLL(path)
    lib.la_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    for kind, iters, grid, out_ in ((0, 0, 8, FAKE), (0, 8, 0, FAKE), (2, 8, 8, FAKE), (1, 8, 8, None)):
        assert lib.la_probe_mfma(kind, iters, grid, out_, None) == -1
    lib.la_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                  ctypes.c_void_p]
    for x, n16, reps, grid, out_ in ((None, 8, 1, 8, FAKE), (FAKE, 0, 1, 8, FAKE), (FAKE, 8, 0, 8, FAKE),
                                     (FAKE, 8, 1, 0, FAKE), (FAKE, 8, 1, 8, None), (0x1008, 8, 1, 8, FAKE)):
        assert lib.la_probe_read(x, n16, reps, grid, out_, None) == -1


def test_version_and_status_strings():
    lib = la.lib()
    assert lib.la_version() >= 100
    for code, text in ((0, b"ok"), (1, b"invalid argument"), (2, b"unsupported"), (3, b"HIP runtime error"),
                       (4, b"workspace missing or too small")):
        assert lib.la_status_string(code) == text
    assert lib.la_status_string(99) == b"unknown status"


def _fwd(**kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, in_dt=b.LA_BF16, BH=2, L=64, d_in=64, d_v=64, C=64, causal=1,
                normalize=0, f=0, W=None, m=0, in_scale=1.0, o=FAKE, out_dt=b.LA_BF16, S_final=None,
                z_final=None, group=0, ws=None, ws_bytes=0, stream=None)
    args.update(kw)
    lib = la.lib()
    return lib.la_chunked_forward(*args.values())


def test_forward_argument_errors():
    lib = la.lib()
    assert _fwd(q=None) == b.LA_ERR_INVALID_ARG
    assert b"NULL" in lib.la_last_error()
    assert _fwd(L=0) == b.LA_ERR_INVALID_ARG
    assert _fwd(BH=-1) == b.LA_ERR_INVALID_ARG
    assert _fwd(d_in=48) == b.LA_ERR_UNSUPPORTED
    assert _fwd(d_v=512) == b.LA_ERR_UNSUPPORTED
    assert _fwd(d_in=8) == b.LA_ERR_UNSUPPORTED
    assert _fwd(in_dt=b.LA_I8, normalize=1, out_dt=b.LA_I32) == b.LA_ERR_UNSUPPORTED
    assert _fwd(in_dt=b.LA_I8, f=1, out_dt=b.LA_I32) == b.LA_ERR_UNSUPPORTED
    assert _fwd(in_dt=b.LA_I8, out_dt=b.LA_BF16) == b.LA_ERR_UNSUPPORTED
    assert _fwd(in_dt=b.LA_I8, out_dt=b.LA_I32, in_scale=0.5) == b.LA_ERR_UNSUPPORTED
    assert _fwd(out_dt=b.LA_I32) == b.LA_ERR_UNSUPPORTED
    assert _fwd(in_dt=b.LA_F32) == b.LA_ERR_UNSUPPORTED
    assert _fwd(f=2, W=None, m=256) == b.LA_ERR_INVALID_ARG  # FAVOR+ without W
    assert _fwd(f=2, W=FAKE, m=100) == b.LA_ERR_UNSUPPORTED
    assert _fwd(f=7) == b.LA_ERR_INVALID_ARG
    assert _fwd(z_final=FAKE) == b.LA_ERR_INVALID_ARG  # z_final needs normalize
    assert _fwd(in_scale=float("nan")) == b.LA_ERR_INVALID_ARG


def test_workspace_sizes_and_errors():
    lib = la.lib()
    ws = lambda *a: lib.la_chunked_forward_workspace(*a)  # noqa: E731
    # one group (group >= N), identity map: no scratch
    assert ws(b.LA_BF16, 128, 8192, 128, 128, 64, 1, 0, 0, 0, 1.0, 1 << 30) == 0
    assert ws(b.LA_BF16, 128, 8192, 128, 128, 64, 1, 0, 0, 0, 0.5, 1 << 30) == 0  # scale folded into the results
    # automatic plan at the headline size, chunks of 64: the streaming kernel's
    # 128 heads x 2 column tiles already fill the GPU, one group per head
    assert ws(b.LA_BF16, 128, 8192, 128, 128, 64, 1, 0, 0, 0, 1.0, 0) == 0
    assert lib.la_chunked_forward_group(b.LA_BF16, 128, 8192, 128, 128, 64, 1, 0, 0, 0, 0) == 8192 // 64
    # chunks of 32 and 128 stream the same way: one group per head
    assert ws(b.LA_BF16, 128, 8192, 128, 128, 32, 1, 0, 0, 0, 1.0, 0) == 0
    assert ws(b.LA_BF16, 128, 8192, 128, 128, 128, 1, 0, 0, 0, 1.0, 0) == 0
    # chunks of 48 (general kernel): four groups of 43 chunks per (head, column
    # tile); phase 1 sums the first three in two pieces of 1032 rows each
    assert ws(b.LA_BF16, 128, 8192, 128, 128, 48, 1, 0, 0, 0, 1.0, 0) == 128 * 4 * 2 * 128 * 128 * 4
    # chunks of 32 keep an even number per group on the streaming kernel
    assert lib.la_chunked_forward_group(b.LA_BF16, 2, 8192, 128, 128, 32, 1, 0, 0, 0, 0) % 2 == 0
    # groups: BH * n_groups * (dk*dv + dk) floats (normalised), 256-byte aligned pieces
    n = ws(b.LA_BF16, 2, 1024, 64, 64, 64, 1, 1, 0, 0, 1.0, 4)
    groups = 1024 // 64 // 4
    assert n == 2 * groups * 64 * 64 * 4 + 2 * groups * 64 * 4
    # elu+1 (mapped inside the kernels): no mapped copies
    n = ws(b.LA_BF16, 2, 1024, 64, 64, 64, 1, 1, 1, 0, 1.0, 4)
    assert n == 2 * groups * 64 * 64 * 4 + 2 * groups * 64 * 4
    # FAVOR+ with m = 64 (streaming kernel): three mapped copies in front
    n = ws(b.LA_BF16, 2, 1024, 64, 64, 64, 1, 1, 2, 64, 1.0, 4)
    assert n == 3 * 2 * 1024 * 64 * 2 + 2 * groups * 64 * 64 * 4 + 2 * groups * 64 * 4
    # few long groups: phase 1 in pieces of >= 512 rows, four per group here
    # (32 heads x 8 groups x 4 pieces: with a map phase 1 also sums the last
    # group, whose total is the returned final state), every piece a state slot
    n = ws(b.LA_BF16, 32, 65536, 64, 64, 128, 1, 1, 1, 0, 1.0, 0)
    assert lib.la_chunked_forward_group(b.LA_BF16, 32, 65536, 64, 64, 128, 1, 1, 1, 0, 0) == 64
    assert n == 32 * 8 * 4 * 64 * 64 * 4 + 32 * 8 * 4 * 64 * 4
    # the identity map: the last group is never summed, and the streaming phase
    # 1 sums each of the other seven whole (32 x 7 workgroups fill the CUs), with
    # or without the decay: one state slot per group
    n = ws(b.LA_BF16, 32, 65536, 64, 64, 128, 1, 1, 0, 0, 1.0, 0)
    assert n == 32 * 8 * 64 * 64 * 4 + 32 * 8 * 64 * 4
    # elu+1 at d_k = 128: no copies either
    n = ws(b.LA_BF16, 2, 1024, 128, 64, 64, 1, 1, 1, 0, 1.0, 4)
    assert n == 2 * groups * 128 * 64 * 4 + 2 * groups * 128 * 4
    # FAVOR+: three mapped copies (q, k and k's residual) of BH*L*m bf16
    n = ws(b.LA_BF16, 24, 16384, 64, 64, 64, 1, 1, 2, 256, 1.0, 0)
    per = 24 * 16384 * 256 * 2
    assert n >= 3 * per
    # non-causal: one total state per head
    assert ws(b.LA_BF16, 3, 100, 64, 32, 64, 0, 0, 0, 0, 1.0, 0) == 3 * 64 * 32 * 4
    # invalid combination
    assert ws(b.LA_BF16, 0, 100, 64, 64, 64, 1, 0, 0, 0, 1.0, 0) == 0
    # too small a workspace is rejected before any launch
    assert _fwd(BH=2, L=1024, normalize=1, f=1, group=4, ws=None, ws_bytes=0) == b.LA_ERR_WORKSPACE
    assert _fwd(BH=2, L=1024, normalize=1, f=1, group=4, ws=FAKE, ws_bytes=100) == b.LA_ERR_WORKSPACE


def test_other_entry_point_errors():
    lib = la.lib()
    assert lib.la_feature_map(0, None, b.LA_BF16, 10, 64, None, 0, 1.0, FAKE, b.LA_BF16, None) == b.LA_ERR_INVALID_ARG
    assert lib.la_feature_map(0, FAKE, b.LA_I8, 10, 64, None, 0, 1.0, FAKE, b.LA_BF16, None) == b.LA_ERR_UNSUPPORTED
    assert lib.la_feature_map(2, FAKE, b.LA_BF16, 10, 64, None, 256, 1.0, FAKE, b.LA_BF16, None) == b.LA_ERR_INVALID_ARG
    assert lib.la_feature_map(1, FAKE, b.LA_BF16, 0, 64, None, 0, 1.0, FAKE, b.LA_BF16, None) == b.LA_ERR_INVALID_ARG
    assert lib.la_chunk_states(None, FAKE, b.LA_BF16, 1, 64, 64, 64, 16, FAKE, None, None) == b.LA_ERR_INVALID_ARG
    assert lib.la_chunk_states(FAKE, FAKE, b.LA_BF16, 1, 64, 24, 64, 16, FAKE, None, None) == b.LA_ERR_UNSUPPORTED
    assert lib.la_chunk_states(FAKE, FAKE, b.LA_F32, 1, 64, 64, 64, 16, FAKE, None, None) == b.LA_ERR_UNSUPPORTED
    assert lib.la_state_scan(None, None, b.LA_F32, 1, 4, 64, 64, None, None, None) == b.LA_ERR_INVALID_ARG
    assert lib.la_state_scan(FAKE, None, b.LA_BF16, 1, 4, 64, 64, None, None, None) == b.LA_ERR_UNSUPPORTED
    assert lib.la_state_scan(FAKE, None, b.LA_F32, 1, 0, 64, 64, None, None, None) == b.LA_ERR_INVALID_ARG
    assert lib.la_state_scan(FAKE, None, b.LA_F32, 1, 4, 64, 64, None, FAKE, None) == b.LA_ERR_INVALID_ARG
    assert lib.la_recurrent_step(FAKE, FAKE, FAKE, b.LA_BF16, 4, 64, 64, 1, None, 0, 1.0, 1, FAKE, None, FAKE,
                                 b.LA_F32, None) == b.LA_ERR_INVALID_ARG  # normalise without z
    assert lib.la_recurrent_step(FAKE, FAKE, FAKE, b.LA_BF16, 4, 64, 64, 2, None, 256, 1.0, 1, FAKE, FAKE, FAKE,
                                 b.LA_F32, None) == b.LA_ERR_INVALID_ARG  # FAVOR+ without W
    assert lib.la_recurrent_step(FAKE, FAKE, FAKE, b.LA_I8, 4, 64, 64, 0, None, 0, 1.0, 0, FAKE, None, FAKE,
                                 b.LA_F32, None) == b.LA_ERR_UNSUPPORTED
    assert lib.la_recurrent_step(FAKE, FAKE, FAKE, b.LA_BF16, 4, 48, 64, 0, None, 0, 1.0, 0, FAKE, None, FAKE,
                                 b.LA_F32, None) == b.LA_ERR_UNSUPPORTED


def test_chunk_output_argument_errors():
    lib = la.lib()
    co = lambda **kw: lib.la_chunk_output(*dict(dict(q=FAKE, k=FAKE, v=FAKE, dt=b.LA_BF16, BH=2, L=256, dk=64, dv=64,
                                                     C=64, group=1, P=None, z=None, norm=0, o=FAKE,
                                                     odt=b.LA_BF16, Sf=None, zf=None, s=None), **kw).values())  # noqa: E731
    assert co(q=None) == b.LA_ERR_INVALID_ARG
    assert co(group=0) == b.LA_ERR_INVALID_ARG
    assert co(group=2, P=None) == b.LA_ERR_INVALID_ARG  # two groups need the prefixes
    assert co(group=2, P=FAKE, norm=1, z=None) == b.LA_ERR_INVALID_ARG
    assert co(dk=96) == b.LA_ERR_UNSUPPORTED
    assert co(dt=b.LA_I8, norm=1, odt=b.LA_I32) == b.LA_ERR_UNSUPPORTED
    assert co(zf=FAKE) == b.LA_ERR_INVALID_ARG


def test_last_error_is_thread_local():
    import threading
    lib = la.lib()
    _fwd(q=None)
    seen = {}

    def other():
        seen["msg"] = lib.la_last_error()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == b""
    assert lib.la_last_error() != b""


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(b, "_lib", None)
    monkeypatch.setattr(b, "LIB_PATH", "/nonexistent/liblinattn.so")
    with pytest.raises(b.LibraryNotBuilt):
        b.lib()


def test_decay_entry_point_errors():
    """The decayed recurrence's entry points: gamma outside (0, 1] or NaN, cases
    off the streaming kernel and wrong phase arguments are rejected up front."""
    lib = la.lib()

    def fwd(gamma=0.9, **kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, in_dt=b.LA_BF16, BH=2, L=64, d_in=64, d_v=64, C=64, normalize=0, f=0,
                 W=None, m=0, in_scale=1.0, o=FAKE, out_dt=b.LA_BF16, S_final=None, z_final=None, group=0,
                 ws=None, ws_bytes=0, stream=None)
        a.update(kw)
        return lib.la_chunked_forward_decay(a["q"], a["k"], a["v"], a["in_dt"], a["BH"], a["L"], a["d_in"], a["d_v"],
                                            a["C"], a["normalize"], a["f"], a["W"], a["m"], a["in_scale"], gamma,
                                            a["o"], a["out_dt"], a["S_final"], a["z_final"], a["group"], a["ws"],
                                            a["ws_bytes"], a["stream"])
    for g in (0.0, -0.5, 1.5, float("nan"), float("inf")):
        assert fwd(gamma=g) == b.LA_ERR_INVALID_ARG, g
    assert fwd(C=48) == b.LA_ERR_UNSUPPORTED            # not a streaming chunk size
    assert fwd(d_in=32) == b.LA_ERR_UNSUPPORTED         # feature width off the streaming kernel
    assert fwd(d_v=32) == b.LA_ERR_UNSUPPORTED          # value width off the streaming kernel
    assert fwd(out_dt=b.LA_F32) == b.LA_ERR_UNSUPPORTED  # fp32 output runs on the general kernel
    assert fwd(in_dt=b.LA_I8, out_dt=b.LA_I32) == b.LA_ERR_UNSUPPORTED
    assert b"streaming" in lib.la_last_error()
    assert lib.la_chunk_states_decay(FAKE, FAKE, b.LA_BF16, 1, 64, 64, 64, 16, 2.0, FAKE, None, None) == \
        b.LA_ERR_INVALID_ARG
    assert lib.la_chunk_states_decay(FAKE, FAKE, b.LA_I8, 1, 64, 64, 64, 16, 0.5, FAKE, None, None) == \
        b.LA_ERR_UNSUPPORTED
    assert lib.la_state_scan_decay(FAKE, None, b.LA_F32, 1, 5, 64, 64, 64, 16, 0.5, None, None, None) == \
        b.LA_ERR_INVALID_ARG  # N != ceil(L / C)
    assert lib.la_state_scan_decay(FAKE, None, b.LA_I32, 1, 4, 64, 64, 64, 16, 0.5, None, None, None) == \
        b.LA_ERR_UNSUPPORTED
    assert lib.la_chunk_output_decay(FAKE, FAKE, FAKE, b.LA_BF16, 1, 40, 64, 64, 48, 1, None, None, 0, 0.5, FAKE,
                                     b.LA_BF16, None, None, None) == b.LA_ERR_UNSUPPORTED
    assert lib.la_recurrent_step_decay(FAKE, FAKE, FAKE, b.LA_BF16, 4, 64, 64, 0, None, 0, 1.0, 0, 0.0, FAKE, None,
                                       FAKE, b.LA_F32, None) == b.LA_ERR_INVALID_ARG


def test_loglinear_entry_point_errors():
    """Log-linear attention: level count, workspace size and argument checks."""
    lib = la.lib()
    assert [lib.la_loglinear_levels(L) for L in (0, 1, 2, 3, 8, 9, 8192)] == [0, 1, 2, 3, 4, 5, 14]
    # 128 heads x 8192 rows, d = 128: 128 chunk states + 64 + 32 + ... + 1 = 127 bucket sums per head
    ws = lib.la_loglinear_forward_workspace(b.LA_BF16, 128, 8192, 128, 128, 64)
    assert ws == 128 * 128 * 128 * 128 * 4 + 128 * 127 * 128 * 128 * 2  # fp32 chunk states, bf16 bucket sums
    assert lib.la_loglinear_forward_workspace(b.LA_BF16, 2, 64, 64, 64, 64) == 0  # one chunk
    assert lib.la_loglinear_forward_workspace(b.LA_BF16, 2, 1000, 64, 64, 32) == 0  # unsupported chunk size

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, in_dt=b.LA_BF16, BH=2, L=1000, d_k=64, d_v=64, C=64, lam=FAKE,
                 n_lev=lib.la_loglinear_levels(1000), o=FAKE, out_dt=b.LA_BF16, S_lev=None, n_slev=0, ws=None,
                 ws_bytes=0)
        a.update(kw)
        return lib.la_loglinear_forward(a["q"], a["k"], a["v"], a["in_dt"], a["BH"], a["L"], a["d_k"], a["d_v"],
                                        a["C"], a["lam"], a["n_lev"], a["o"], a["out_dt"], a["S_lev"], a["n_slev"],
                                        a["ws"], a["ws_bytes"], None)
    assert call(lam=None) == b.LA_ERR_INVALID_ARG
    assert call(n_lev=5) == b.LA_ERR_INVALID_ARG
    # the level states: n_state_levels from la_loglinear_levels(L) (11 here) to 40, read only with S_levels
    assert call(S_lev=FAKE, n_slev=10) == b.LA_ERR_INVALID_ARG
    assert call(S_lev=FAKE, n_slev=41) == b.LA_ERR_INVALID_ARG
    assert call(S_lev=FAKE, n_slev=11) == b.LA_ERR_WORKSPACE
    assert call(S_lev=None, n_slev=-3) == b.LA_ERR_WORKSPACE
    assert call(C=32) == b.LA_ERR_UNSUPPORTED
    assert call(d_k=32) == b.LA_ERR_UNSUPPORTED
    assert call(d_v=32) == b.LA_ERR_UNSUPPORTED
    assert call(in_dt=b.LA_I8) == b.LA_ERR_UNSUPPORTED
    assert call(out_dt=b.LA_F32) == b.LA_ERR_UNSUPPORTED
    assert call() == b.LA_ERR_WORKSPACE


def test_loglinear_step_entry_point_errors():
    """The log-linear decode step: NULL pointers, sizes, a negative position,
    too few (or more than 40) levels for the position, types and widths are
    rejected before any launch."""
    lib = la.lib()

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, in_dt=b.LA_BF16, n=3, d_k=64, d_v=64, lam=FAKE, n_lev=4, t=7, S=FAKE,
                 o=FAKE, out_dt=b.LA_F32)
        a.update(kw)
        return lib.la_recurrent_step_loglinear(a["q"], a["k"], a["v"], a["in_dt"], a["n"], a["d_k"], a["d_v"],
                                               a["lam"], a["n_lev"], a["t"], a["S"], a["o"], a["out_dt"], None)
    for name in ("q", "k", "v", "lam", "S", "o"):
        assert call(**{name: None}) == b.LA_ERR_INVALID_ARG, name
    assert call(n=0) == b.LA_ERR_INVALID_ARG
    assert call(t=-1) == b.LA_ERR_INVALID_ARG
    assert call(t=8, n_lev=4) == b.LA_ERR_INVALID_ARG  # position 8 needs 5 levels
    assert call(t=0, n_lev=0) == b.LA_ERR_INVALID_ARG
    assert call(t=0, n_lev=41) == b.LA_ERR_INVALID_ARG
    assert call(in_dt=b.LA_I8) == b.LA_ERR_UNSUPPORTED
    assert call(out_dt=b.LA_I32) == b.LA_ERR_UNSUPPORTED
    assert call(d_k=48) == b.LA_ERR_UNSUPPORTED
    assert call(d_v=512) == b.LA_ERR_UNSUPPORTED


def test_delta_entry_point_errors():
    """The delta rule: workspace size (per-chunk 64 x 64 bf16 transforms and the
    gates' log products) and argument checks, all before any launch."""
    lib = la.lib()
    ws = lib.la_chunked_forward_delta_workspace(b.LA_BF16, 128, 8192, 128, 128, 64)
    assert ws == 128 * 128 * 64 * 64 * 2 + 128 * 128 * 64 * 4
    assert lib.la_chunked_forward_delta_workspace(b.LA_BF16, 2, 100, 64, 64, 64) == 2 * 2 * 8192 + 2 * 2 * 256
    assert lib.la_chunked_forward_delta_workspace(b.LA_BF16, 2, 100, 64, 64, 32) == 0  # chunks of 64 only
    assert lib.la_chunked_forward_delta_workspace(b.LA_BF16, 2, 100, 256, 64, 64) == 0
    assert lib.la_chunked_forward_delta_workspace(b.LA_I8, 2, 100, 64, 64, 64) == 0

    def fwd(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, in_dt=b.LA_BF16, BH=2, L=100, d_k=64, d_v=64, C=64, beta=FAKE, alpha=None,
                 o=FAKE, out_dt=b.LA_BF16, S=None, ws=FAKE, ws_bytes=0)
        a.update(kw)
        return lib.la_chunked_forward_delta(a["q"], a["k"], a["v"], a["in_dt"], a["BH"], a["L"], a["d_k"], a["d_v"],
                                            a["C"], a["beta"], a["alpha"], a["o"], a["out_dt"], a["S"], a["ws"],
                                            a["ws_bytes"], None)
    assert fwd(beta=None) == b.LA_ERR_INVALID_ARG
    assert fwd(L=0) == b.LA_ERR_INVALID_ARG
    assert fwd(C=128) == b.LA_ERR_UNSUPPORTED
    assert fwd(d_k=32) == b.LA_ERR_UNSUPPORTED
    assert fwd(d_v=32) == b.LA_ERR_UNSUPPORTED
    assert fwd(in_dt=b.LA_I8) == b.LA_ERR_UNSUPPORTED
    assert fwd(out_dt=b.LA_F32) == b.LA_ERR_UNSUPPORTED
    assert fwd(ws_bytes=100) == b.LA_ERR_WORKSPACE
    assert b"workspace" in lib.la_last_error()
    assert lib.la_delta_chunk_transform(FAKE, None, None, b.LA_BF16, 2, 100, 64, 64, FAKE, FAKE, None) == \
        b.LA_ERR_INVALID_ARG
    assert lib.la_delta_chunk_transform(FAKE, FAKE, None, b.LA_BF16, 2, 100, 64, 16, FAKE, FAKE, None) == \
        b.LA_ERR_UNSUPPORTED

    def step(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, in_dt=b.LA_BF16, n=4, d_k=64, d_v=64, beta=FAKE, alpha=None, S=FAKE, o=FAKE,
                 out_dt=b.LA_F32)
        a.update(kw)
        return lib.la_recurrent_step_delta(a["q"], a["k"], a["v"], a["in_dt"], a["n"], a["d_k"], a["d_v"], a["beta"],
                                           a["alpha"], a["S"], a["o"], a["out_dt"], None)
    assert step(S=None) == b.LA_ERR_INVALID_ARG
    assert step(n=0) == b.LA_ERR_INVALID_ARG
    assert step(d_k=48) == b.LA_ERR_UNSUPPORTED
    assert step(d_v=512) == b.LA_ERR_UNSUPPORTED
    assert step(out_dt=b.LA_I32) == b.LA_ERR_UNSUPPORTED
    assert step(in_dt=b.LA_F32) == b.LA_ERR_UNSUPPORTED


def test_loglinear_prefix_levels_entry_point_errors():
    """The log-linear prefix levels: workspace (the states of the whole 64-row
    chunks before the last row's chunk) and argument checks before any launch."""
    lib = la.lib()
    assert lib.la_loglinear_prefix_levels_workspace(b.LA_BF16, 2, 64, 64, 64) == 0  # one chunk
    assert lib.la_loglinear_prefix_levels_workspace(b.LA_BF16, 2, 65, 64, 64) == 2 * 1 * 64 * 64 * 4
    assert lib.la_loglinear_prefix_levels_workspace(b.LA_BF16, 128, 8192, 128, 128) == 128 * 127 * 128 * 128 * 4
    assert lib.la_loglinear_prefix_levels_workspace(b.LA_I8, 2, 100, 64, 64) == 0  # unsupported

    def call(**kw):
        a = dict(k=FAKE, v=FAKE, in_dt=b.LA_BF16, BH=2, L=1000, d_k=64, d_v=64, n_lev=lib.la_loglinear_levels(1000),
                 S=FAKE, ws=None, ws_bytes=0)
        a.update(kw)
        return lib.la_loglinear_prefix_levels(a["k"], a["v"], a["in_dt"], a["BH"], a["L"], a["d_k"], a["d_v"],
                                              a["n_lev"], a["S"], a["ws"], a["ws_bytes"], None)
    for name in ("k", "v", "S"):
        assert call(**{name: None}) == b.LA_ERR_INVALID_ARG, name
    assert call(L=0) == b.LA_ERR_INVALID_ARG
    assert call(n_lev=lib.la_loglinear_levels(1000) - 1) == b.LA_ERR_INVALID_ARG
    assert call(n_lev=41) == b.LA_ERR_INVALID_ARG
    assert call(in_dt=b.LA_I8) == b.LA_ERR_UNSUPPORTED
    assert call(d_k=48) == b.LA_ERR_UNSUPPORTED
    assert call() == b.LA_ERR_WORKSPACE


def test_int8_step_entry_point_errors():
    """The exact int8 decode step: NULL pointers, sizes, widths and a misaligned
    state are rejected before any launch."""
    lib = la.lib()

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, n=3, d_k=16, d_v=16, S=FAKE, o=FAKE)
        a.update(kw)
        return lib.la_recurrent_step_i8(a["q"], a["k"], a["v"], a["n"], a["d_k"], a["d_v"], a["S"], a["o"], None)
    for name in ("q", "k", "v", "S", "o"):
        assert call(**{name: None}) == b.LA_ERR_INVALID_ARG, name
    assert call(n=0) == b.LA_ERR_INVALID_ARG
    assert call(S=0x1004) == b.LA_ERR_INVALID_ARG
    assert call(d_k=24) == b.LA_ERR_UNSUPPORTED
    assert call(d_v=512) == b.LA_ERR_UNSUPPORTED
