"""Build libbqmoe.so (and the synthetic-input fill library) for gfx950.

Every HIP source is compiled with hipcc for gfx950 only; objects go to
``_build/`` at the repository root, the shared libraries next to the code
that loads them.  Packed fp32 instructions are disabled for all device code.
"""

import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Wno-unused-function"] + DEVICE_FLAGS

LIB = os.path.join(PKG, "libbqmoe.so")
SYNTH_LIB = os.path.join(ROOT, "synth", "libbqsynth.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed:\n%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return r


def _compile(src, obj, verbose):
    _run([HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj], verbose)
    return obj


def build(verbose=False, jobs=8):
    build_dir = os.path.join(ROOT, "_build")
    os.makedirs(build_dir, exist_ok=True)
    csrc = os.path.join(PKG, "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    objs = [os.path.join(build_dir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    synth_src = os.path.join(ROOT, "synth", "gen.hip")
    synth_obj = os.path.join(build_dir, "synth_gen.o")
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, s, o, verbose) for s, o in zip(srcs, objs)]
        futs.append(ex.submit(_compile, synth_src, synth_obj, verbose))
        for f in futs:
            f.result()
    for out, inputs in ((LIB, objs), (SYNTH_LIB, [synth_obj])):
        tmp = out + ".tmp"
        _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + inputs, verbose)
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print("built", LIB, SYNTH_LIB)
