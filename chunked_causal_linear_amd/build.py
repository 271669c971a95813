"""Build liblinattn.so (HIP, gfx950) in-tree.

Compiles every ``csrc/*.hip`` translation unit with hipcc in parallel into
``_build/`` and links ``chunked_causal_linear_amd/liblinattn.so``; the
measurement probe (``csrc/probe/*.hip``, a matrix-core rate loop) goes into
``libla_probe.so`` beside it.  The build runs on a machine without a GPU
(hipcc cross-compiles for gfx950).

    python -m chunked_causal_linear_amd.build            # rebuild everything
    python -m chunked_causal_linear_amd.build --changed  # only stale objects
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblinattn.so")
PROBE_LIB = os.path.join(PKG, "libla_probe.so")
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# -packed-fp32-ops: keep the compiler from emitting packed fp32 vector ops.
CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I" + INCLUDE, "-I" + CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Per-file flags.  The streaming kernel keeps its matrix-core accumulators in
# ordinary VGPRs (it runs one wave per SIMD, so all 512 registers are there),
# which saves the copies out of accumulation registers before every pack; so
# does the FAVOR+ map, whose epilogue reads every accumulator once.  The
# variants with the most live registers (la_pipe_wide.hip) are built without
# it: that form fails to compile at their register pressure.
FILE_FLAGS = {"la_pipe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "la_pipe_decay.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "la_pipe_decay_fac.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "la_fmap.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "la_delta.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "la_favor.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "probe/la_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def _probe_sources():
    return sorted("probe/" + f for f in os.listdir(os.path.join(CSRC, "probe")) if f.endswith(".hip"))


def _headers_mtime() -> float:
    hs = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")]
    hs += [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h")]
    return max(os.path.getmtime(h) for h in hs)


def _compile(src: str) -> tuple:
    obj = os.path.join(BUILD, src[:-4].replace("/", "_") + ".o")
    cmd = [HIPCC] + CFLAGS + FILE_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    err = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    return src, r.returncode, err, time.time() - t0


def build(changed_only: bool = False, jobs: int = None, verbose: bool = True) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    probe_srcs = _probe_sources()
    todo = []
    hdr_t = _headers_mtime()
    for s in srcs + probe_srcs:
        obj = os.path.join(BUILD, s[:-4].replace("/", "_") + ".o")
        if changed_only and os.path.exists(obj):
            ot = os.path.getmtime(obj)
            if ot >= os.path.getmtime(os.path.join(CSRC, s)) and ot >= hdr_t:
                continue
        todo.append(s)
    jobs = jobs or min(len(todo) or 1, max(1, (os.cpu_count() or 4)))
    failed = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, rc, err, dt in ex.map(_compile, todo):
            if verbose:
                print(f"[build] {src}: {'ok' if rc == 0 else 'FAILED'} ({dt:.1f}s)", flush=True)
            if rc != 0:
                failed.append((src, err))
            elif err.strip() and verbose:
                print(err, flush=True)
    if failed:
        msg = "\n".join(f"--- {s}\n{e}" for s, e in failed)
        raise RuntimeError("HIP build failed:\n" + msg)
    for lib, group in ((LIB, srcs), (PROBE_LIB, probe_srcs)):
        objs = [os.path.join(BUILD, s[:-4].replace("/", "_") + ".o") for s in group]
        tmp = lib + ".tmp"
        cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stderr)
        os.replace(tmp, lib)
        if verbose:
            print(f"[build] linked {lib}", flush=True)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--changed", action="store_true", help="recompile only stale objects")
    ap.add_argument("-j", type=int, default=None)
    a = ap.parse_args(argv)
    build(changed_only=a.changed, jobs=a.j)


if __name__ == "__main__":
    sys.exit(main())
