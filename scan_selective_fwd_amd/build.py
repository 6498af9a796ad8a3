"""Builds the HIP library libmamba_scan.so for gfx950 with hipcc.

Every source under csrc/ is compiled to an object in parallel, then linked
into scan_selective_fwd_amd/libmamba_scan.so.  HIP code is built with packed
FP32 instructions disabled (`-Xclang -target-feature -Xclang -packed-fp32-ops`).

`python -m scan_selective_fwd_amd.build --incremental` recompiles only the
objects whose source or included headers changed (hipcc -MMD dependency
files); build() without it recompiles everything.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmamba_scan.so")
ARCH = os.environ.get("MAMBA_SCAN_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _up_to_date(obj):
    dep = obj + ".d"
    if not (os.path.exists(obj) and os.path.exists(dep)):
        return False
    with open(dep) as f:
        text = f.read().replace("\\\n", " ")
    deps = text.split(":", 1)[1].split() if ":" in text else []
    t = os.path.getmtime(obj)
    return all(os.path.exists(d) and os.path.getmtime(d) <= t for d in deps)


def _compile(src, verbose, incremental=False):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if incremental and _up_to_date(obj):
        return obj
    cmd = [HIPCC] + COMMON + ["-MMD", "-MF", obj + ".d", "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + [f for f in COMMON if f not in ("-Xclang", "-target-feature",
                                                        "-packed-fp32-ops")] + [
            "-MMD", "-MF", obj + ".d", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed for {src}")
    return obj


def build(verbose: bool = False, jobs: int = 8, incremental: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, incremental), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    t = __import__("time").time()
    print(build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv))
    print(f"built in {__import__('time').time() - t:.1f}s")
