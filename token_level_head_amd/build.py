"""Build libmhla.so (the HIP library for gfx950) in-tree with hipcc.

    python -m token_level_head_amd.build
    python -m token_level_head_amd.build --resources   # per-kernel registers, scratch, LDS (markdown)
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
           "bwd_fused.hip", "mhla_api.hip"]
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
    ("bwd_fused", "bwd_fused.hip"),
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


def resources():
    """Markdown table of every kernel's resource usage, from the compiler's
    kernel-resource-usage remarks (device code only, the library's own flags)."""
    import re

    rows = []
    for src in SOURCES:
        r = subprocess.run([HIPCC, *FLAGS, "--cuda-device-only", "-Rpass-analysis=kernel-resource-usage", "-c",
                            os.path.join(CSRC, src), "-o", os.devnull], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(r.stderr[-2000:])
        cur = None
        for line in r.stderr.splitlines():
            m = re.search(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                          r"VGPRs Spill|LDS Size \[bytes/block\]): (\S+)", line)
            if not m:
                continue
            key, val = m.groups()
            if key == "Function Name":
                cur = {"kernel": _demangle(val), "source": src}
                rows.append(cur)
            elif cur is not None:
                cur[key] = val
    out = ["| kernel | source | VGPRs | AGPRs | VGPR spills | scratch B/lane | LDS B | waves/SIMD |", "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{r['kernel']}` | {r['source']} | {r.get('VGPRs')} | {r.get('AGPRs')} | {r.get('VGPRs Spill')} | "
                   f"{r.get('ScratchSize [bytes/lane]')} | {r.get('LDS Size [bytes/block]')} | {r.get('Occupancy [waves/SIMD]')} |")
    return "\n".join(out)


def _demangle(name):
    for tool in ("c++filt", "llvm-cxxfilt"):
        try:
            r = subprocess.run([tool, name], capture_output=True, text=True)
        except OSError:
            continue
        if r.returncode == 0 and r.stdout.strip():
            name = r.stdout.strip()
            break
    return name.replace("(anonymous namespace)::", "").replace("mhla::", "").split("(")[0].replace("void ", "")


if __name__ == "__main__":
    if "--resources" in sys.argv:
        print(f"# Kernel resources (gfx950)\n\nCommand: `python -m token_level_head_amd.build --resources`\n\n"
              f"Kernel sources digest: `{source_digest()}`\n")
        print(resources())
    else:
        print(build(verbose=True))
