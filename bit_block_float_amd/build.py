"""Build libhif4.so (the HIP library for gfx950) in-tree with hipcc.

Usage: python -m bit_block_float_amd.build   (or import and call build()).
The library is compiled for gfx950 only. Packed fp32 VALU instructions are
disabled in the device pass (-packed-fp32-ops); the host pass warns that it
does not know that feature, which is harmless.
"""
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhif4.so")
SOURCES = ["api.hip", "quant.hip", "gemm.hip", "pct.hip", "gptq.hip", "autoround.hip"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def hipcc() -> str:
    p = os.path.join(ROCM, "bin", "hipcc")
    return p if os.path.exists(p) else (shutil.which("hipcc") or "hipcc")


def flags():
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        "-Wall", "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(os.path.dirname(HERE), "include"),
    ]


PROBE_LIB = os.path.join(HERE, "libhif4_probe.so")


def build_probe(verbose: bool = False) -> str:
    """Compile libhif4_probe.so (measurement probes used by bench.py --ceilings)."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), *flags(), "-shared", os.path.join(CSRC, "probe.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    text = "\n".join(l for l in p.stdout.decode(errors="replace").splitlines()
                     if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for probe.hip:\n{text}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source to an object, then link libhif4.so (and the probe
    library). Always rebuilds."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    for p in procs:
        _wait(p, verbose)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    build_probe(verbose)
    return LIB


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # drop the host pass's harmless "unknown feature" notes
    text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{text}")
    if verbose and text.strip():
        print(text)


if __name__ == "__main__":
    print(build(verbose=True))
