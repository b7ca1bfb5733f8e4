"""Build the HIP C-ABI library ``libmoe_hip.so`` for gfx950 in-tree.

Every translation unit under ``csrc/`` is compiled by hipcc (in parallel) and
linked into one shared library next to this file.  Flags:
  --offload-arch=gfx950          MI355X only
  -O3 -ffp-contract=off          no implicit FMA contraction (the routing score
                                 is a fixed sequence of IEEE operations)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                 no packed-fp32 instructions
  -Werror=inline-asm             inline assembly must not clobber reserved
                                 registers (the LDS copies save and restore M0)
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_hip.so")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Werror=inline-asm"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# host-code sanitizers (AddressSanitizer + UndefinedBehaviorSanitizer) for a
# CPU-only check of the argument validation: each flag applies to the host
# compilation only (-Xarch_host), the device code is built as usual
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def _compile(src, verbose, build_dir=BUILD, extra=()):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False, lib: str = LIB, build_dir: str = BUILD,
          sanitize: bool = False) -> str:
    """Compile every csrc/*.hip and link `lib`.  sanitize: host code under
    AddressSanitizer and UndefinedBehaviorSanitizer (the library then needs
    clang's ASan runtime preloaded; see tests/test_sanitizers.py)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    extra = HOST_SANITIZE if sanitize else ()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
