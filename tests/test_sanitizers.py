"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (``oracle/mhla_oracle.c``) is rebuilt with gcc's ASan + UBSan and every
  pin of ``tests/oracle_pins.py`` runs through it; two copies with a planted mistake
  (a heap write one past a buffer, a signed overflow) show that the sanitizers report
  such errors in this set-up.
* The host side of the C ABI (argument validation, workspace bookkeeping, the
  allocation-failure path) is rebuilt with clang's ASan + UBSan -- host code only;
  the device code is built as usual -- and the host-only ABI and binding tests run
  against that build.

No GPU is used: the ABI tests make no call that reaches a device.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "oracle_pins.py")
CSRC = os.path.join(ROOT, "token_level_head_amd", "csrc")
ROCM = "/opt/rocm"


def _gcc_runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _clang_asan_runtime():
    found = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    return found[-1] if found else None


GCC_ASAN = _gcc_runtime("libasan.so")
CLANG_ASAN = _clang_asan_runtime()
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0", "UBSAN_OPTIONS": "print_stacktrace=1"}


def _build_oracle(tmp_path, name, edit=None):
    work = tmp_path / name
    work.mkdir()
    text = open(os.path.join(ROOT, "oracle", "mhla_oracle.c")).read()
    if edit is not None:
        old, new = edit
        assert text.count(old) == 1, f"site for {name} no longer unique in mhla_oracle.c"
        text = text.replace(old, new)
    (work / "mhla_oracle.c").write_text(text)
    shutil.copy(os.path.join(ROOT, "oracle", "mhla_oracle.h"), work / "mhla_oracle.h")
    lib = str(work / "lib.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    str(work / "mhla_oracle.c"), "-o", lib, "-lm"], check=True)
    return lib


def _run_pins(lib):
    env = dict(os.environ, LD_PRELOAD=GCC_ASAN, **SAN_ENV)
    return subprocess.run([sys.executable, PINS, "--lib", lib], capture_output=True, text=True, timeout=600,
                          env=env)


def _reports(r):
    text = r.stdout + r.stderr
    return "AddressSanitizer" in text or "runtime error" in text


needs_gcc_asan = pytest.mark.skipif(GCC_ASAN is None, reason="gcc's libasan is not installed")


@needs_gcc_asan
def test_oracle_pins_clean_under_sanitizers(tmp_path):
    r = _run_pins(_build_oracle(tmp_path, "clean"))
    assert r.returncode == 0 and not _reports(r), r.stdout[-3000:] + r.stderr[-3000:]


@needs_gcc_asan
def test_planted_heap_overflow_is_reported(tmp_path):
    # phi(k) written one element past its d-element buffer
    edit = ("for (long r = 0; r < d; ++r) fk[r] = mhla_oracle_phi((double)kj[r]);",
            "for (long r = 0; r <= d; ++r) fk[r] = mhla_oracle_phi((double)kj[r]);")
    r = _run_pins(_build_oracle(tmp_path, "overflow", edit))
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]


@needs_gcc_asan
def test_planted_signed_overflow_is_reported(tmp_path):
    edit = ("    const long C = N / M;\n    double* fk = (double*)malloc(sizeof(double) * d);",
            "    const long C = N / M;\n    volatile int big = 0x7fffffff;\n"
            "    if (big + (int)N == 0) return -1;\n"
            "    double* fk = (double*)malloc(sizeof(double) * d);")
    r = _run_pins(_build_oracle(tmp_path, "signed_overflow", edit))
    assert r.returncode != 0 and "signed integer overflow" in r.stderr, r.stderr[-3000:]


def _objects():
    """The library's objects as the normal build leaves them (built here if missing)."""
    from token_level_head_amd import build

    objs = [os.path.join(build.OBJDIR, os.path.splitext(s)[0] + ".o") for s in build.SOURCES]
    if not all(os.path.exists(o) for o in objs):
        build.build()
    return build, objs


@pytest.mark.skipif(CLANG_ASAN is None or not os.path.exists(os.path.join(ROCM, "bin", "hipcc")),
                    reason="ROCm's clang sanitizer runtime or hipcc is missing")
def test_host_abi_clean_under_sanitizers(tmp_path):
    build, objs = _objects()
    api_obj = str(tmp_path / "mhla_api_san.o")
    # Sanitizers on the host pass only (-Xarch_host before each -fsanitize=); device code as usual.
    cmd = [build.HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={build.ARCH}",
           "-I", build.INCLUDE, "-I", CSRC, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-c", os.path.join(CSRC, "mhla_api.hip"), "-o", api_obj]
    subprocess.run(cmd, check=True, capture_output=True)
    lib = str(tmp_path / "libmhla_san.so")
    others = [o for o in objs if not o.endswith("mhla_api.o")]
    subprocess.run([os.path.join(ROCM, "llvm", "bin", "clang++"), "-shared", "-shared-libsan",
                    "-fsanitize=address,undefined", "-o", lib, api_obj, *others,
                    f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"], check=True, capture_output=True)
    env = dict(os.environ, LD_PRELOAD=CLANG_ASAN, MHLA_LIBRARY=lib, **SAN_ENV)
    probe = ("import token_level_head_amd as mh; mh.load_library(); "
             "print(any('libmhla_san.so' in l for l in open('/proc/self/maps')))")
    r = subprocess.run([sys.executable, "-c", probe], capture_output=True, text=True, env=env, cwd=ROOT,
                       timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "True", r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_binding_checks.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    assert r.returncode == 0 and not _reports(r), r.stdout[-3000:] + r.stderr[-3000:]
