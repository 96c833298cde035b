"""Build libkascade.so (the gfx950 HIP library behind include/kascade.h) in place."""
import concurrent.futures
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIBRARY = os.path.join(HERE, "libkascade.so")
PROBE_LIBRARY = os.path.join(HERE, "libkascade_probe.so")  # measurement probes used by bench.py --probe
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # Packed fp32 instructions stay off: the compiler keeps to scalar fp32 ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core results in ordinary VGPRs, so the vector ALU reads them
    # without a copy out of the accumulation registers.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # No NaN operands are assumed (inputs are finite; masking uses -inf), so
    # fmaxf needs no NaN-quieting copies of its operands.
    "-fno-honor-nans",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src, build_dir=BUILD, defines=()):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, library):
    tmp = library + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, library)


def build(verbose=False, library=LIBRARY, build_dir=BUILD, defines=(), probe=True):
    """Compile every kernel source for gfx950 and link the shared library, and
    (probe=True) the measurement probe library next to it.

    `defines` (NAME=VALUE strings) and a different `library` path build a
    variant of the library with other compile-time settings."""
    os.makedirs(build_dir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probes = sorted(glob.glob(os.path.join(CSRC, "probe", "*.hip"))) if probe else []
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(sources) + len(probes))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines), sources + probes))
    _link(objs[:len(sources)], library)
    if probes:
        _link(objs[len(sources):], PROBE_LIBRARY)
    if verbose:
        print(library)
    return library


if __name__ == "__main__":
    build(verbose=True)
