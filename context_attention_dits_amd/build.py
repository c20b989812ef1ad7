"""Build the gfx950 HIP library ``libcpattn.so`` in-tree with hipcc.

Usage: ``python -m context_attention_dits_amd.build [--out PATH] [-DNAME=VALUE ...]``.
Every call compiles from source (no up-to-date check). Objects go to
``context_attention_dits_amd/_build/``; the shared library lands next to this
file unless ``--out`` says otherwise. ``-D`` definitions select kernel tile
variants (e.g. ``-DCP_FWD_QB=2``: two 32-query blocks per wave, 4-wave shape only) for a
library built at another path.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import ctypes
import os
import shutil
import subprocess
import sys
from typing import Dict, List, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libcpattn.so"
SOURCES = ["api.hip", "attn_bwd_bf16.hip", "attn_fwd_bf16.hip", "attn_fwd_f32.hip", "lse_merge.hip", "regroup.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU instructions are left out of the generated code on purpose.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


# A second library for the GPU test of the one-launch ring's bounded merge wait: the same
# sources with every merge, after its real wait, waiting 16 polls for a flag no workgroup sets,
# so every wait gives up, is counted and poisons its tile, while every kernel still ends normally.
RING_WAIT_TEST_LIB = "libcpattn_ringwait_test.so"
RING_WAIT_TEST_DEFINES = {"CP_RING_TEST_NEVER_READY": "1"}
# A diagnostic library: the block kernel's one-block launch also records the core-clock cycles of
# its tile-loop intervals (work, wait for tile loads, barrier wait; cp_debug_phase_trace), and a
# synthetic ping-pong with the tile loop's instruction mix and no memory traffic is added
# (cp_debug_mix_probe); the C ABI header declares neither. bench.py --phase-trace loads it.
PHASE_TRACE_LIB = "libcpattn_phase.so"
PHASE_TRACE_DEFINES = {"CP_FWD_PHASE_TRACE": "1"}
# Libraries built next to the main one with only the forward kernel recompiled: name -> defines.
VARIANT_LIBS = {RING_WAIT_TEST_LIB: RING_WAIT_TEST_DEFINES, PHASE_TRACE_LIB: PHASE_TRACE_DEFINES}
# Sources only a variant library links in: name -> sources.
VARIANT_EXTRA_SOURCES = {PHASE_TRACE_LIB: ["diag_mix.hip"]}


def build(out: Optional[str] = None, defines: Optional[Dict[str, str]] = None,
          build_dir: Optional[str] = None, verbose: bool = False, test_libs: bool = True) -> str:
    out = out or os.path.join(PKG, LIB_NAME)
    tag = "_".join(f"{k}{v}" for k, v in sorted((defines or {}).items())) or "default"
    build_dir = build_dir or os.path.join(PKG, "_build", tag)
    os.makedirs(build_dir, exist_ok=True)
    dflags: List[str] = [f"-D{k}={v}" for k, v in sorted((defines or {}).items())]
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        cmd = [cc, *HIPCC_FLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        return obj

    def link(objs: List[str], dst: str) -> None:
        tmp = dst + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        # Resolve every symbol now (RTLD_NOW), so a missing kernel stub fails the build, not the first call.
        try:
            ctypes.CDLL(tmp, mode=os.RTLD_NOW)
        except OSError as e:
            os.remove(tmp)
            raise RuntimeError(f"built library does not load: {e}") from e
        os.replace(tmp, dst)

    # the variant libraries need only the forward kernel recompiled with their defines
    with_variants = test_libs and not defines

    def compile_variant(name: str) -> List[str]:
        """The variant's forward kernel object, then its extra sources' objects."""
        vdir = os.path.join(PKG, "_build", name.replace(".so", ""))
        os.makedirs(vdir, exist_ok=True)
        df = [f"-D{k}={v}" for k, v in sorted(VARIANT_LIBS[name].items())]
        objs = []
        for src in ["attn_fwd_bf16.hip", *VARIANT_EXTRA_SOURCES.get(name, [])]:
            obj = os.path.join(vdir, src.replace(".hip", ".o"))
            cmd = [cc, *HIPCC_FLAGS, *df, "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src} ({name} build):\n{r.stderr}")
            objs.append(obj)
        return objs

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES) + len(VARIANT_LIBS), os.cpu_count() or 4)) as ex:
        futs = [ex.submit(compile_one, src) for src in SOURCES]
        var_futs = {n: ex.submit(compile_variant, n) for n in VARIANT_LIBS} if with_variants else {}
        objs = [f.result() for f in futs]
        var_objs = {n: f.result() for n, f in var_futs.items()}
    link(objs, out)
    for name, vobjs in var_objs.items():
        link([vobjs[0] if os.path.basename(o) == "attn_fwd_bf16.o" else o for o in objs] + vobjs[1:],
             os.path.join(os.path.dirname(out), name))
    return out


# Host-side sanitizers for the C ABI's argument checking (api.hip), host pass only: the GPU code
# is built as usual. The link puts the shared sanitizer runtime on the library's run path; a process
# that is not itself instrumented (python) must preload that runtime (sanitizer_runtime()).
SANITIZE_HOST_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g",
]
SANITIZED_LIB = "libcpattn_sanitized.so"


def _clangxx() -> str:
    return os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang++")


def sanitizer_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the ROCm LLVM toolchain (it carries UBSan too)."""
    r = subprocess.run([_clangxx(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("ROCm LLVM's shared ASan runtime not found")
    return path


def build_sanitized(out_dir: str) -> str:
    """Build ``out_dir/libcpattn_sanitized.so``: api.hip's host code under AddressSanitizer and
    UndefinedBehaviorSanitizer, every other source as in build(). For CPU tests of the host-side
    validation (no kernel is launched by them)."""
    os.makedirs(out_dir, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        extra = SANITIZE_HOST_FLAGS if src == "api.hip" else []
        r = subprocess.run([cc, *HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src} (sanitized build):\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    out = os.path.join(out_dir, SANITIZED_LIB)
    rt_dir = os.path.dirname(sanitizer_runtime())
    rocm_lib = os.path.join(os.path.dirname(os.path.realpath(cc)), "..", "lib")
    link_flags = ["-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan"]
    r = subprocess.run([_clangxx(), *link_flags, "-o", out, *objs, f"-L{rocm_lib}", "-lamdhip64",
                        f"-Wl,-rpath,{rocm_lib}", f"-Wl,-rpath,{rt_dir}"], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--out", default=None)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    defs = {}
    for d in a.defines:
        k, _, v = d.partition("=")
        defs[k] = v or "1"
    path = build(a.out, defs, verbose=a.verbose)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
