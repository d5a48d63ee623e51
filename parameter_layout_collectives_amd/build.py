"""Build libtide.so (the TIDE C-ABI library) for gfx950 with hipcc.

    python -m parameter_layout_collectives_amd.build [--out PATH] [-D NAME=VALUE ...]

-D overrides a tuning macro of the kernels or the launch policy (for
experiments; the in-tree library is always built with the defaults), --out
writes the library elsewhere than the package directory.

Flags:
  * --offload-arch=gfx950: CDNA4 only;
  * -ffp-contract=off, no fast-math: the reduction is a chain of IEEE binary32
    additions with subnormals kept, so results are bit-reproducible;
  * -Xclang -target-feature -Xclang -packed-fp32-ops: no packed fp32 ALU ops
    (hipcc's host pass warns that it does not know the feature; harmless).
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtide.so")

SOURCES = ["plan.cpp", "runtime.hip", "kernels.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose=False, out=LIB, extra=()):
    """Compile every HIP/C++ source into `out` (always rebuilds)."""
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        raise RuntimeError("hipcc not found: the TIDE library needs ROCm to build")
    hipcc = HIPCC if os.path.exists(HIPCC) else shutil.which("hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS, *extra, "-I", INCLUDE,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def main(argv=None):
    import argparse
    ap = argparse.ArgumentParser(description="build libtide.so for gfx950")
    ap.add_argument("--out", default=LIB, help="library path (default: in the package)")
    ap.add_argument("-D", dest="defines", action="append", default=[], metavar="NAME=VALUE",
                    help="override a tuning macro, e.g. -D TIDE_RS_WG_CAP=4")
    args = ap.parse_args(argv)
    for d in args.defines:
        name = d.split("=", 1)[0]
        if not name.startswith("TIDE_") or not name[5:].replace("_", "").isalnum():
            ap.error(f"-D {d}: only TIDE_* tuning macros can be overridden")
    build(verbose=True, out=os.path.abspath(args.out), extra=[f"-D{d}" for d in args.defines])
    return 0


if __name__ == "__main__":
    sys.exit(main())
