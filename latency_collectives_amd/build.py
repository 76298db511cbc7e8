"""Build the HIP library (libar.so) for gfx950 in-tree.

    python -m latency_collectives_amd.build

compiles every ``csrc/*.hip`` file with hipcc into ``latency_collectives_amd/libar.so``.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libar.so")
ARCH = os.environ.get("AR_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Never let the compiler form packed fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile the library unconditionally and return its path. Every source is compiled to an
    object file in its own hipcc process (in parallel), then the objects are linked."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="ar_build_") as d:
        objs = [os.path.join(d, os.path.basename(src) + ".o") for src in sources()]
        cmds = [[hipcc, *compile_flags, "-c", src, "-o", obj]
                for src, obj in zip(sources(), objs)]
        cmds.append([hipcc, *HIPCC_FLAGS, *objs, "-o", tmp])

        def run(cmd):
            if verbose:
                print(" ".join(cmd), flush=True)
            return subprocess.run(cmd, capture_output=True, text=True)

        with ThreadPoolExecutor(max_workers=len(objs)) as pool:
            results = list(pool.map(run, cmds[:-1]))
        results.append(run(cmds[-1]) if all(r.returncode == 0 for r in results) else None)
        for r in results:
            if r is None or r.returncode != 0:
                for q in results:
                    if q is not None:
                        sys.stderr.write(q.stdout + q.stderr)
                raise RuntimeError("hipcc failed to build libar.so")
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    """Build only when no library exists yet (tests and tools call this)."""
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
