"""Build the fp64 CPU oracle (test infrastructure only) with gcc.

`build()` compiles kascade_oracle.c into liboracle shared object next to the
source. `build_variant()` compiles a given C source text elsewhere; the tests
use it to plant deliberate mistakes in a copy of the oracle and check that the
pins catch them.
"""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "kascade_oracle.c")
LIBRARY = os.path.join(HERE, "libkascade_oracle.so")

# Plain IEEE double arithmetic: no fast-math, no contraction into FMA.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def _compile(src_path, out_path):
    tmp = out_path + ".tmp"
    cmd = ["gcc", *CFLAGS, "-I", HERE, src_path, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, out_path)
    return out_path


def build():
    """Compile the oracle library in place and return its path."""
    return _compile(SOURCE, LIBRARY)


def build_variant(source_text, out_dir=None):
    """Compile `source_text` (a modified copy of the oracle) into out_dir."""
    out_dir = out_dir or tempfile.mkdtemp(prefix="oracle_variant_")
    src = os.path.join(out_dir, "variant.c")
    with open(src, "w") as f:
        f.write(source_text)
    return _compile(src, os.path.join(out_dir, "libvariant.so"))


def read_source():
    with open(SOURCE) as f:
        return f.read()


if __name__ == "__main__":
    print(build())
