"""Build libmhla.so (the HIP library for gfx950) in-tree with hipcc.

    python -m token_level_head_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmhla.so")
SOURCES = ["summary.hip", "mix.hip", "output.hip", "causal.hip", "decode.hip", "backward.hip", "fused.hip", "pair.hip",
           "mhla_api.hip"]
OBJDIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 instructions are kept out of the generated code on purpose.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result"]


# The source file that defines each kernel family (by kernel-name prefix); a
# kernel's measurements stay valid while this file and the shared headers do.
KERNEL_SOURCES = [
    ("fused_", "fused.hip"),
    ("pair_", "pair.hip"),
    ("summaries_", "summary.hip"),
    ("mix_", "mix.hip"),
    ("wsplit_", "mix.hip"),
    ("output_causal_quad", "causal.hip"),
    ("output_", "output.hip"),
    ("decode_", "decode.hip"),
    ("bwd_", "backward.hip"),
]
SHARED_SOURCES = ["common.hpp", "kernels.hpp", "lds_tiles.hpp", "mhla_api.hip", "../../include/mhla.h"]


def source_digest(files=None):
    """SHA-256 (first 16 hex digits) over kernel and ABI sources: identifies which
    code a profile measured.  Without `files`, every source of the library."""
    import hashlib

    if files is None:
        files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp"))) + ["../../include/mhla.h"]
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def kernel_source_digest(kernel_name):
    """Digest of the file defining `kernel_name` plus the shared headers, or of all
    sources when the name matches no known family."""
    base = kernel_name.replace("mhla::", "").replace("void ", "").strip()
    for prefix, src in KERNEL_SOURCES:
        if base.startswith(prefix):
            return source_digest([src] + SHARED_SOURCES)
    return source_digest()


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is expected.
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    return err


def build(verbose=False, out=LIB):
    os.makedirs(OBJDIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        msg = _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj, msg

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for _, msg in results:
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
    tmp = out + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *[o for o, _ in results]])
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
