"""Build libspecverify.so (the HIP/gfx950 library) in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspecverify.so")
SOURCES = ["api.hip", "attn.hip", "accept.hip", "multidraft.hip", "commit.hip", "tree.hip", "linattn.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose=False):
    """Compile every HIP source into libspecverify.so (always recompiles).

    SPEC_HOST_FLAGS (whitespace-separated) adds flags for the host side, each
    passed behind -Xarch_host so device code is untouched; the CPU sanitizer
    run (tests/sanitize_cpu.sh) uses it."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    host = []
    for f in os.environ.get("SPEC_HOST_FLAGS", "").split():
        host += ["-Xarch_host", f]
    cmd = [HIPCC, *FLAGS, *host, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
