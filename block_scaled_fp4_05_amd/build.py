"""Compile the HIP library (libmoe_fp4.so) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_fp4.so")
SOURCES = ["api.cpp", "quantize.hip", "grouped_gemm.hip", "grouped_gemm_finalize.hip",
           "grouped_gemm_swiglu.hip", "grouped_gemm_tiled.hip", "grouped_gemm_big.hip", "grouped_gemm_mid.hip", "pack.hip", "combine.hip"]
HEADERS = ["fp4_device.h", "gemm_common.h", "grouped_gemm_kernel.h", "launch.h"]
# A measurement aid kept out of the library: the streaming-read probe that
# bench.py --ceilings loads (not part of the C ABI in include/moe_fp4.h).
PROBE_LIB = os.path.join(PKG, "libmoe_fp4_probe.so")
PROBE_SOURCES = ["stream_probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # Keep the compiler from forming packed-FP32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Device code must round every float operation as written.
    "-ffp-contract=off", "-fno-fast-math",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, out: str | None = None, extra_flags=(), sources=None) -> str:
    """Always recompiles (each source to an object in parallel, then one link);
    writes the library atomically to `out` (default: the in-tree library).
    `extra_flags` go on every compile and the link (the host-sanitizer build of
    the CPU tests passes -Xarch_host flags here).  `sources` defaults to the
    library's; build_probe() passes the probe's."""
    out = out or LIB
    srcs = list(sources or SOURCES)
    from concurrent.futures import ThreadPoolExecutor
    import tempfile

    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="moe_fp4_build_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [cc, *[f for f in HIPCC_FLAGS if f != "-shared"], *extra_flags, *inc, "-c",
                   os.path.join(CSRC, src), "-o", obj]
            return obj, subprocess.run(cmd, capture_output=True, text=True)

        workers = max(1, min(len(srcs), os.cpu_count() or 1, 8))
        with ThreadPoolExecutor(max_workers=workers) as pool:
            results = list(pool.map(compile_one, srcs))
        log = []
        for (obj, res), src in zip(results, srcs):
            log.append(res.stdout + res.stderr)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n" + res.stdout + res.stderr)
        tmp = out + ".tmp%d" % os.getpid()
        link = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *extra_flags,
                *[o for o, _ in results], "-o", tmp]
        res = subprocess.run(link, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
        if verbose:
            print("".join(log) + res.stderr)
        os.replace(tmp, out)
    return out


def build_probe(verbose: bool = False) -> str:
    """The streaming-read probe library (libmoe_fp4_probe.so)."""
    return build(verbose=verbose, out=PROBE_LIB, sources=PROBE_SOURCES)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))
