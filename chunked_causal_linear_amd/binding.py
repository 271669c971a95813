"""Thin Python binding of liblinattn's C ABI (``include/la.h``).

Argument marshalling only: every wrapper checks the torch tensors it is handed
(device, dtype, shape, contiguity), passes their device pointers and the
current HIP stream to the library, and raises on a non-OK status.  All the
arithmetic runs in the library's HIP kernels; there is no fallback.  The
library is loaded on first use and a missing or unloadable library raises
``LibraryNotBuilt``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblinattn.so")

# la_status
LA_OK, LA_ERR_INVALID_ARG, LA_ERR_UNSUPPORTED, LA_ERR_HIP, LA_ERR_WORKSPACE = range(5)
# la_dtype
LA_BF16, LA_F32, LA_I8, LA_I32 = range(4)
# la_fmap
FMAPS = {"identity": 0, "elu1": 1, "favor": 2}

EXPORTS = (
    "la_feature_map", "la_chunk_states", "la_state_scan", "la_chunk_output", "la_chunked_forward",
    "la_chunked_forward_workspace", "la_chunked_forward_group", "la_recurrent_step", "la_status_string", "la_last_error",
    "la_version", "la_chunk_states_decay", "la_state_scan_decay", "la_chunk_output_decay", "la_chunked_forward_decay",
    "la_recurrent_step_decay", "la_loglinear_forward", "la_loglinear_forward_workspace", "la_loglinear_levels",
    "la_chunked_forward_delta", "la_chunked_forward_delta_workspace", "la_delta_chunk_transform",
    "la_recurrent_step_delta", "la_chunked_forward_noalloc", "la_recurrent_step_loglinear",
    "la_loglinear_prefix_levels", "la_loglinear_prefix_levels_workspace", "la_recurrent_step_i8",
)


class LibraryNotBuilt(RuntimeError):
    pass


class LAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"liblinattn status {status}: {message}")
        self.status = status


_lib = None


def _declare(lib: ctypes.CDLL) -> None:
    i64, f32, vp, i32, sz = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.la_feature_map.argtypes = [i32, vp, i32, i64, i64, vp, i64, f32, vp, i32, vp]
    lib.la_chunk_states.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, vp, vp, vp]
    lib.la_state_scan.argtypes = [vp, vp, i32, i64, i64, i64, i64, vp, vp, vp]
    lib.la_chunk_output.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, i64, vp, vp, i32, vp, i32, vp, vp, vp]
    lib.la_chunked_forward.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, i32, i32, i32, vp, i64, f32,
                                       vp, i32, vp, vp, i64, vp, sz, vp]
    lib.la_chunked_forward_workspace.argtypes = [i32, i64, i64, i64, i64, i64, i32, i32, i32, i64, f32, i64]
    lib.la_chunked_forward_workspace.restype = sz
    lib.la_chunked_forward_group.argtypes = [i32, i64, i64, i64, i64, i64, i32, i32, i32, i64, i64]
    lib.la_chunked_forward_group.restype = i64
    lib.la_recurrent_step.argtypes = [vp, vp, vp, i32, i64, i64, i64, i32, vp, i64, f32, i32, vp, vp, vp, i32, vp]
    # the decayed recurrence: the same arguments with gamma
    lib.la_chunk_states_decay.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, f32, vp, vp, vp]
    lib.la_state_scan_decay.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, i64, f32, vp, vp, vp]
    lib.la_chunk_output_decay.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, i64, vp, vp, i32, f32, vp, i32,
                                          vp, vp, vp]
    lib.la_chunked_forward_decay.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, i32, i32, vp, i64, f32, f32,
                                             vp, i32, vp, vp, i64, vp, sz, vp]
    lib.la_recurrent_step_decay.argtypes = [vp, vp, vp, i32, i64, i64, i64, i32, vp, i64, f32, i32, f32, vp, vp, vp,
                                            i32, vp]
    lib.la_loglinear_forward.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, vp, i64, vp, i32, vp, i64, vp, sz, vp]
    lib.la_loglinear_forward_workspace.argtypes = [i32, i64, i64, i64, i64, i64]
    lib.la_loglinear_forward_workspace.restype = sz
    lib.la_loglinear_levels.argtypes = [i64]
    lib.la_loglinear_levels.restype = i64
    lib.la_recurrent_step_loglinear.argtypes = [vp, vp, vp, i32, i64, i64, i64, vp, i64, i64, vp, vp, i32, vp]
    lib.la_loglinear_prefix_levels.argtypes = [vp, vp, i32, i64, i64, i64, i64, i64, vp, vp, sz, vp]
    lib.la_recurrent_step_i8.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp]
    lib.la_loglinear_prefix_levels_workspace.argtypes = [i32, i64, i64, i64, i64]
    lib.la_loglinear_prefix_levels_workspace.restype = sz
    lib.la_chunked_forward_delta.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, vp, vp, vp, i32, vp, vp, sz,
                                             vp]
    lib.la_chunked_forward_delta_workspace.argtypes = [i32, i64, i64, i64, i64, i64]
    lib.la_chunked_forward_delta_workspace.restype = sz
    lib.la_delta_chunk_transform.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, vp, vp, vp]
    lib.la_recurrent_step_delta.argtypes = [vp, vp, vp, i32, i64, i64, i64, vp, vp, vp, vp, i32, vp]
    lib.la_chunked_forward_noalloc.argtypes = [vp, vp, vp, i32, i64, i64, i64, i64, i64, i32, i32, i32, vp, i64, f32,
                                               vp, i32, vp, vp, i64, vp]
    for name in ("la_chunked_forward_noalloc", "la_chunked_forward_delta", "la_delta_chunk_transform", "la_recurrent_step_delta",
                 "la_loglinear_forward", "la_feature_map", "la_chunk_states", "la_state_scan", "la_chunk_output",
                 "la_chunked_forward",
                 "la_recurrent_step", "la_chunk_states_decay", "la_state_scan_decay", "la_chunk_output_decay",
                 "la_chunked_forward_decay", "la_recurrent_step_decay"):
        getattr(lib, name).restype = i32
    lib.la_status_string.argtypes = [i32]
    lib.la_status_string.restype = ctypes.c_char_p
    lib.la_last_error.argtypes = []
    lib.la_last_error.restype = ctypes.c_char_p
    lib.la_version.argtypes = []
    lib.la_version.restype = i32


def lib() -> ctypes.CDLL:
    """The loaded library (loads it on first call)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryNotBuilt(f"{LIB_PATH} is missing: build it with "
                                  "`python -m chunked_causal_linear_amd.build`")
        try:
            handle = ctypes.CDLL(LIB_PATH)
        except OSError as e:
            raise LibraryNotBuilt(f"cannot load {LIB_PATH}: {e}") from e
        _declare(handle)
        _lib = handle
    return _lib


def _check(status: int) -> None:
    if status != LA_OK:
        msg = lib().la_last_error().decode("utf-8", "replace")
        raise LAError(status, msg or lib().la_status_string(status).decode())


# ---------------------------------------------------------------------------
# torch helpers (device memory and streams only)
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_ptr() -> int:
    torch = _torch()
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.bfloat16: LA_BF16, torch.float32: LA_F32, torch.int8: LA_I8, torch.int32: LA_I32}
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def _dev(t, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _fmap_code(fmap: str) -> int:
    if fmap not in FMAPS:
        raise ValueError(f"fmap must be one of {sorted(FMAPS)}")
    return FMAPS[fmap]


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def feature_map(x, fmap: str, W=None, in_scale: float = 1.0, out_dtype=None, out=None):
    """phi(in_scale * x) row by row; x [..., d_in] bf16 -> [..., d_k] (into `out` if given)."""
    torch = _torch()
    d_in = x.shape[-1]
    rows = x.numel() // d_in
    m = W.shape[0] if (fmap == "favor" and W is not None) else 0
    d_k = m if fmap == "favor" else d_in
    y = out if out is not None else torch.empty(*x.shape[:-1], d_k, dtype=out_dtype or torch.bfloat16,
                                                device=x.device)
    if tuple(y.shape) != tuple(x.shape[:-1]) + (d_k,):
        raise ValueError(f"out has shape {tuple(y.shape)}, expected {tuple(x.shape[:-1]) + (d_k,)}")
    _check(lib().la_feature_map(_fmap_code(fmap), _dev(x, "x"), _dtype_code(x), rows, d_in,
                                _dev(W, "W"), m, float(in_scale), _dev(y, "y"), _dtype_code(y), _stream_ptr()))
    return y


def chunk_states(k, v, C: int, want_z: bool = False, out=None, gamma: float = 1.0):
    """Phase 1: per-chunk states S [BH, N, d_k, d_v] (and z [BH, N, d_k]); `out` = S to reuse.
    gamma != 1: the decayed recurrence's states at each chunk's end."""
    torch = _torch()
    BH, L, d_k = k.shape
    d_v = v.shape[-1]
    Cs = 1 if C <= 0 else min(C, L)
    N = (L + Cs - 1) // Cs
    st = torch.int32 if k.dtype == torch.int8 else torch.float32
    S = out if out is not None else torch.empty(BH, N, d_k, d_v, dtype=st, device=k.device)
    if tuple(S.shape) != (BH, N, d_k, d_v) or S.dtype != st:
        raise ValueError(f"out must be {(BH, N, d_k, d_v)} {st}")
    z = torch.empty(BH, N, d_k, dtype=st, device=k.device) if want_z else None
    if gamma != 1.0:
        _check(lib().la_chunk_states_decay(_dev(k, "k"), _dev(v, "v"), _dtype_code(k), BH, L, d_k, d_v, C,
                                           float(gamma), _dev(S, "S"), _dev(z, "z"), _stream_ptr()))
    else:
        _check(lib().la_chunk_states(_dev(k, "k"), _dev(v, "v"), _dtype_code(k), BH, L, d_k, d_v, C,
                                     _dev(S, "S"), _dev(z, "z"), _stream_ptr()))
    return S, z


def state_scan(S, z=None, want_final: bool = True, gamma: float = 1.0, L: int = 0, C: int = 0):
    """Phase 2, in place: S (and z) become exclusive prefixes; returns (S_final, z_final).
    gamma != 1: the decayed prefix over chunks of C rows of an L-row sequence."""
    torch = _torch()
    BH, N, d_k, d_v = S.shape
    Sf = torch.empty(BH, d_k, d_v, dtype=S.dtype, device=S.device) if want_final else None
    zf = torch.empty(BH, d_k, dtype=S.dtype, device=S.device) if (want_final and z is not None) else None
    if gamma != 1.0:
        _check(lib().la_state_scan_decay(_dev(S, "S"), _dev(z, "z"), _dtype_code(S), BH, N, d_k, d_v, L, C,
                                         float(gamma), _dev(Sf, "S_final"), _dev(zf, "z_final"), _stream_ptr()))
    else:
        _check(lib().la_state_scan(_dev(S, "S"), _dev(z, "z"), _dtype_code(S), BH, N, d_k, d_v,
                                   _dev(Sf, "S_final"), _dev(zf, "z_final"), _stream_ptr()))
    return Sf, zf


def chunk_output(q, k, v, C: int, group: int, P_prefix=None, z_prefix=None, normalize: bool = False,
                 out_dtype=None, return_state: bool = False, out=None, gamma: float = 1.0):
    """Phase 3 alone from group prefix states (see la_chunk_output; gamma != 1: la_chunk_output_decay)."""
    torch = _torch()
    BH, L, d_k = q.shape
    d_v = v.shape[-1]
    i8 = q.dtype == torch.int8
    if out is None:
        out = torch.empty(BH, L, d_v, dtype=out_dtype or (torch.int32 if i8 else torch.bfloat16), device=q.device)
    st = torch.int32 if i8 else torch.float32
    Sf = torch.empty(BH, d_k, d_v, dtype=st, device=q.device) if return_state else None
    zf = torch.empty(BH, d_k, dtype=torch.float32, device=q.device) if (return_state and normalize) else None
    if gamma != 1.0:
        _check(lib().la_chunk_output_decay(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dtype_code(q), BH, L, d_k,
                                           d_v, C, group, _dev(P_prefix, "P_prefix"), _dev(z_prefix, "z_prefix"),
                                           int(normalize), float(gamma), _dev(out, "o"), _dtype_code(out),
                                           _dev(Sf, "S_final"), _dev(zf, "z_final"), _stream_ptr()))
    else:
        _check(lib().la_chunk_output(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dtype_code(q), BH, L, d_k, d_v, C,
                                     group, _dev(P_prefix, "P_prefix"), _dev(z_prefix, "z_prefix"), int(normalize),
                                     _dev(out, "o"), _dtype_code(out), _dev(Sf, "S_final"), _dev(zf, "z_final"),
                                     _stream_ptr()))
    if return_state:
        return out, Sf, zf
    return out


def forward_workspace_bytes(in_dtype_code: int, BH: int, L: int, d_in: int, d_v: int, C: int, causal: bool,
                            normalize: bool, fmap: str, m: int = 0, in_scale: float = 1.0, group: int = 0) -> int:
    return int(lib().la_chunked_forward_workspace(in_dtype_code, BH, L, d_in, d_v, C, int(causal), int(normalize),
                                                  _fmap_code(fmap), m, float(in_scale), group))


def forward_group(in_dtype_code: int, BH: int, L: int, d_in: int, d_v: int, C: int, causal: bool,
                  normalize: bool, fmap: str, m: int = 0, group: int = 0) -> int:
    """Chunks per group la_chunked_forward uses for these arguments."""
    return int(lib().la_chunked_forward_group(in_dtype_code, BH, L, d_in, d_v, C, int(causal), int(normalize),
                                              _fmap_code(fmap), m, group))


class Forward:
    """A planned forward call with its output, final-state and workspace buffers.

    Allocate once (``__init__``), then ``run()`` enqueues only the library's
    kernels on the current stream - the form the benchmark times.
    """

    def __init__(self, q, k, v, C: int, causal: bool = True, normalize: bool = False, fmap: str = "identity",
                 W=None, in_scale: float = 1.0, out_dtype=None, return_state: bool = False, group: int = 0,
                 gamma: float = 1.0):
        torch = _torch()
        self.gamma = float(gamma)
        self.q, self.k, self.v, self.W = q, k, v, W
        BH, L, d_in = q.shape
        d_v = v.shape[-1]
        self.m = W.shape[0] if (fmap == "favor" and W is not None) else 0
        d_k = self.m if fmap == "favor" else d_in
        self.shape = (BH, L, d_in, d_v, d_k)
        self.C, self.causal, self.normalize, self.fmap = C, causal, normalize, fmap
        self.in_scale, self.group = float(in_scale), group
        i8 = q.dtype == torch.int8
        if out_dtype is None:
            out_dtype = torch.int32 if i8 else torch.bfloat16
        self.o = torch.empty(BH, L, d_v, dtype=out_dtype, device=q.device)
        st = torch.int32 if i8 else torch.float32
        self.S_final = torch.empty(BH, d_k, d_v, dtype=st, device=q.device) if return_state else None
        self.z_final = (torch.empty(BH, d_k, dtype=torch.float32, device=q.device)
                        if (return_state and normalize) else None)
        ws = forward_workspace_bytes(_dtype_code(q), BH, L, d_in, d_v, C, causal, normalize, fmap, self.m,
                                     self.in_scale, group)
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=q.device)
        self.ws_bytes = ws
        for name, t in (("q", q), ("k", k), ("v", v), ("W", W)):
            _dev(t, name)

    def run(self):
        BH, L, d_in, d_v, _ = self.shape
        if self.gamma != 1.0:
            if not self.causal:
                raise ValueError("the decayed recurrence is causal")
            _check(lib().la_chunked_forward_decay(
                self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), _dtype_code(self.q), BH, L, d_in, d_v,
                self.C, int(self.normalize), _fmap_code(self.fmap),
                self.W.data_ptr() if self.W is not None else None, self.m, self.in_scale, self.gamma,
                self.o.data_ptr(), _dtype_code(self.o),
                self.S_final.data_ptr() if self.S_final is not None else None,
                self.z_final.data_ptr() if self.z_final is not None else None,
                self.group, self.workspace.data_ptr(), self.ws_bytes, _stream_ptr()))
            return self.o
        _check(lib().la_chunked_forward(
            self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), _dtype_code(self.q), BH, L, d_in, d_v,
            self.C, int(self.causal), int(self.normalize), _fmap_code(self.fmap),
            self.W.data_ptr() if self.W is not None else None, self.m, self.in_scale,
            self.o.data_ptr(), _dtype_code(self.o),
            self.S_final.data_ptr() if self.S_final is not None else None,
            self.z_final.data_ptr() if self.z_final is not None else None,
            self.group, self.workspace.data_ptr(), self.ws_bytes, _stream_ptr()))
        return self.o


def chunked_forward(q, k, v, C: int, causal: bool = True, normalize: bool = False, fmap: str = "identity",
                    W=None, in_scale: float = 1.0, out_dtype=None, return_state: bool = False,
                    group: int = 0, gamma: float = 1.0) -> Tuple:
    """O (and, with return_state, the final S and z) of the chunked forward (gamma != 1: the decayed
    recurrence, la_chunked_forward_decay)."""
    f = Forward(q, k, v, C, causal, normalize, fmap, W, in_scale, out_dtype, return_state, group, gamma)
    o = f.run()
    if return_state:
        return o, f.S_final, f.z_final
    return o


def loglinear_levels(L: int) -> int:
    """Levels la_loglinear_forward uses for L tokens (1 + bit length of L - 1)."""
    return int(lib().la_loglinear_levels(L))


class LogLinearForward:
    """A planned log-linear forward (chunks of 64) with its output and workspace."""

    def __init__(self, q, k, v, lam, C: int = 64, state_levels: Optional[int] = None):
        """state_levels: also write the level states after the last token (see
        la_loglinear_forward's S_levels) with that many levels, into self.S_levels."""
        torch = _torch()
        BH, L, d_k = q.shape
        d_v = v.shape[-1]
        self.q, self.k, self.v, self.lam, self.C = q, k, v, lam, C
        self.shape = (BH, L, d_k, d_v)
        if lam.dtype != torch.float32 or tuple(lam.shape) != (BH, L, loglinear_levels(L)):
            raise ValueError(f"lam must be float32 {(BH, L, loglinear_levels(L))}")
        self.o = torch.empty(BH, L, d_v, dtype=torch.bfloat16, device=q.device)
        self.n_state_levels = 0 if state_levels is None else int(state_levels)
        self.S_levels = None
        if state_levels is not None:
            self.S_levels = torch.empty(BH, self.n_state_levels, d_k, d_v, dtype=torch.float32, device=q.device)
        ws = int(lib().la_loglinear_forward_workspace(_dtype_code(q), BH, L, d_k, d_v, C))
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=q.device)
        self.ws_bytes = ws
        for name, t in (("q", q), ("k", k), ("v", v), ("lam", lam)):
            _dev(t, name)

    def run(self):
        BH, L, d_k, d_v = self.shape
        _check(lib().la_loglinear_forward(self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(),
                                          _dtype_code(self.q), BH, L, d_k, d_v, self.C, self.lam.data_ptr(),
                                          self.lam.shape[-1], self.o.data_ptr(), _dtype_code(self.o),
                                          self.S_levels.data_ptr() if self.S_levels is not None else None,
                                          self.n_state_levels, self.workspace.data_ptr(), self.ws_bytes,
                                          _stream_ptr()))
        return self.o


def loglinear_forward(q, k, v, lam, C: int = 64, return_levels: bool = False, n_state_levels: Optional[int] = None):
    """Log-linear attention output (see la_loglinear_forward); lam [BH, L, levels] float32.
    With return_levels, returns (o, S_levels): also the level states after the last
    token [BH, n_state_levels, d_k, d_v] float32 (n_state_levels defaults to
    loglinear_levels(L); pass more to decode past a power of two)."""
    if not return_levels:
        return LogLinearForward(q, k, v, lam, C).run()
    n = loglinear_levels(q.shape[1]) if n_state_levels is None else n_state_levels
    f = LogLinearForward(q, k, v, lam, C, state_levels=n)
    return f.run(), f.S_levels


def recurrent_step_i8(q, k, v, S, out=None):
    """One exact int8 decode step (la_recurrent_step_i8) over n states: q, k [n, d_k],
    v [n, d_v] int8; S [n, d_k, d_v] int32 updates in place; returns o [n, d_v] int32."""
    torch = _torch()
    n, d_k = q.shape
    d_v = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.int8:
            raise ValueError(f"{name} must be int8")
    if S.dtype != torch.int32 or tuple(S.shape) != (n, d_k, d_v):
        raise ValueError(f"S must be int32 {(n, d_k, d_v)}")
    if out is None:
        out = torch.empty(n, d_v, dtype=torch.int32, device=q.device)
    _check(lib().la_recurrent_step_i8(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), n, d_k, d_v, _dev(S, "S"),
                                      _dev(out, "o"), _stream_ptr()))
    return out


def loglinear_prefix_levels(k, v, n_levels: Optional[int] = None):
    """The level states after the L tokens of k, v [BH, L, d] (bf16): what decode
    steps at positions 0 .. L - 1 from zero states leave (la_loglinear_prefix_levels).
    Returns S [BH, n_levels, d_k, d_v] float32; n_levels defaults to
    loglinear_levels(L) (pass more to continue decoding past a power of two)."""
    torch = _torch()
    BH, L, d_k = k.shape
    d_v = v.shape[-1]
    n_lev = loglinear_levels(L) if n_levels is None else int(n_levels)
    S = torch.empty(BH, n_lev, d_k, d_v, dtype=torch.float32, device=k.device)
    ws = int(lib().la_loglinear_prefix_levels_workspace(_dtype_code(k), BH, L, d_k, d_v))
    work = torch.empty(max(ws, 1), dtype=torch.uint8, device=k.device)
    _check(lib().la_loglinear_prefix_levels(_dev(k, "k"), _dev(v, "v"), _dtype_code(k), BH, L, d_k, d_v, n_lev,
                                            _dev(S, "S"), work.data_ptr(), ws, _stream_ptr()))
    return S


def recurrent_step_loglinear(q, k, v, lam, S, t: int, out=None):
    """One log-linear decode step (la_recurrent_step_loglinear) at position t over
    n streams: q, k [n, d_k], v [n, d_v] bf16; lam [n, levels] float32 (this
    token's level weights); S [n, levels, d_k, d_v] float32 updates in place."""
    torch = _torch()
    n, d_k = q.shape
    d_v = v.shape[-1]
    if lam.dtype != torch.float32 or lam.dim() != 2 or lam.shape[0] != n:
        raise ValueError(f"lam must be float32 [{n}, levels]")
    n_lev = lam.shape[1]
    if S.dtype != torch.float32 or tuple(S.shape) != (n, n_lev, d_k, d_v):
        raise ValueError(f"S must be float32 {(n, n_lev, d_k, d_v)}")
    if out is None:
        out = torch.empty(n, d_v, dtype=torch.float32, device=q.device)
    _check(lib().la_recurrent_step_loglinear(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dtype_code(q), n, d_k, d_v,
                                             _dev(lam, "lam"), n_lev, int(t), _dev(S, "S"), _dev(out, "o"),
                                             _dtype_code(out), _stream_ptr()))
    return out


def recurrent_step(q, k, v, S, z=None, fmap: str = "identity", W=None, in_scale: float = 1.0,
                   normalize: bool = True, out=None, gamma: float = 1.0):
    """One decode step over n states; S [n, d_k, d_v] and z [n, d_k] (fp32) update in place
    (gamma != 1: S = gamma S + phi(k) v^T, la_recurrent_step_decay)."""
    torch = _torch()
    n, d_in = q.shape
    d_v = v.shape[-1]
    m = W.shape[0] if (fmap == "favor" and W is not None) else 0
    if out is None:
        out = torch.empty(n, d_v, dtype=torch.float32, device=q.device)
    if gamma != 1.0:
        _check(lib().la_recurrent_step_decay(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dtype_code(q), n, d_in,
                                             d_v, _fmap_code(fmap), _dev(W, "W"), m, float(in_scale),
                                             int(normalize), float(gamma), _dev(S, "S"), _dev(z, "z"),
                                             _dev(out, "o"), _dtype_code(out), _stream_ptr()))
    else:
        _check(lib().la_recurrent_step(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dtype_code(q), n, d_in, d_v,
                                       _fmap_code(fmap), _dev(W, "W"), m, float(in_scale), int(normalize),
                                       _dev(S, "S"), _dev(z, "z"), _dev(out, "o"), _dtype_code(out), _stream_ptr()))
    return out


# ---------------------------------------------------------------------------
# the delta rule (include/la.h: la_chunked_forward_delta and its companions)
# ---------------------------------------------------------------------------
def _gates(beta, alpha, shape, device):
    torch = _torch()
    for name, t in (("beta", beta), ("alpha", alpha)):
        if t is None:
            continue
        if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must be float32 {tuple(shape)}")
        _dev(t, name)


class DeltaForward:
    """A planned delta-rule forward (chunks of 64) with its output, final-state
    and workspace buffers; ``run()`` enqueues only the library's kernels."""

    def __init__(self, q, k, v, beta, alpha=None, C: int = 64, return_state: bool = False):
        torch = _torch()
        BH, L, d_k = q.shape
        d_v = v.shape[-1]
        _gates(beta, alpha, (BH, L), q.device)
        self.q, self.k, self.v, self.beta, self.alpha, self.C = q, k, v, beta, alpha, C
        self.shape = (BH, L, d_k, d_v)
        self.o = torch.empty(BH, L, d_v, dtype=torch.bfloat16, device=q.device)
        self.S_final = torch.empty(BH, d_k, d_v, dtype=torch.float32, device=q.device) if return_state else None
        ws = int(lib().la_chunked_forward_delta_workspace(_dtype_code(q), BH, L, d_k, d_v, C))
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=q.device)
        self.ws_bytes = ws
        for name, t in (("q", q), ("k", k), ("v", v)):
            _dev(t, name)

    def run(self):
        BH, L, d_k, d_v = self.shape
        _check(lib().la_chunked_forward_delta(
            self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), _dtype_code(self.q), BH, L, d_k, d_v, self.C,
            self.beta.data_ptr(), self.alpha.data_ptr() if self.alpha is not None else None, self.o.data_ptr(),
            _dtype_code(self.o), self.S_final.data_ptr() if self.S_final is not None else None,
            self.workspace.data_ptr(), self.ws_bytes, _stream_ptr()))
        return self.o


def delta_forward(q, k, v, beta, alpha=None, C: int = 64, return_state: bool = False):
    """O (and, with return_state, the final state) of the (gated) delta rule; beta, alpha [BH, L] float32."""
    f = DeltaForward(q, k, v, beta, alpha, C, return_state)
    o = f.run()
    return (o, f.S_final) if return_state else o


def delta_chunk_transform(k, beta, alpha=None, C: int = 64):
    """Per-chunk T [BH, N, 64, 64] (bf16, columns in operand order) and gate log products lg [BH, N, 64]."""
    torch = _torch()
    BH, L, d_k = k.shape
    _gates(beta, alpha, (BH, L), k.device)
    N = (L + 63) // 64
    T = torch.empty(BH, N, 64, 64, dtype=torch.bfloat16, device=k.device)
    lg = torch.empty(BH, N, 64, dtype=torch.float32, device=k.device)
    _check(lib().la_delta_chunk_transform(_dev(k, "k"), _dev(beta, "beta"), _dev(alpha, "alpha"), _dtype_code(k), BH,
                                          L, d_k, C, _dev(T, "T"), _dev(lg, "lg"), _stream_ptr()))
    return T, lg


def recurrent_step_delta(q, k, v, S, beta, alpha=None, out=None):
    """One (gated) delta-rule decode step over n states; S [n, d_k, d_v] fp32 updates in place."""
    torch = _torch()
    n, d_k = q.shape
    d_v = v.shape[-1]
    _gates(beta, alpha, (n,), q.device)
    if out is None:
        out = torch.empty(n, d_v, dtype=torch.float32, device=q.device)
    _check(lib().la_recurrent_step_delta(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dtype_code(q), n, d_k, d_v,
                                         _dev(beta, "beta"), _dev(alpha, "alpha"), _dev(S, "S"), _dev(out, "o"),
                                         _dtype_code(out), _stream_ptr()))
    return out


def chunked_forward_noalloc(q, k, v, C: int, causal: bool = True, normalize: bool = False, fmap: str = "identity",
                            W=None, in_scale: float = 1.0, out=None, S_final=None, z_final=None, group: int = 0):
    """la_chunked_forward_noalloc: the forward with the library's own static scratch
    (no workspace).  Writes into `out` (and `S_final`, `z_final` when given) and
    returns out."""
    torch = _torch()
    BH, L, d_in = q.shape
    d_v = v.shape[-1]
    m = W.shape[0] if (fmap == "favor" and W is not None) else 0
    if out is None:
        out = torch.empty(BH, L, d_v, dtype=torch.bfloat16, device=q.device)
    _check(lib().la_chunked_forward_noalloc(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dtype_code(q), BH, L, d_in, d_v,
                                            C, int(causal), int(normalize), _fmap_code(fmap), _dev(W, "W"), m,
                                            float(in_scale), _dev(out, "o"), _dtype_code(out),
                                            _dev(S_final, "S_final"), _dev(z_final, "z_final"), group,
                                            _stream_ptr()))
    return out
