"""CPU runs under AddressSanitizer and UndefinedBehaviorSanitizer (host code
only): the oracle's pin suites against an instrumented build of the oracle,
and the C ABI's host-side checks against an instrumented build of the
library's host runtime.  A planted one-byte heap overflow in a copy of the
oracle shows that the instrumented runs do catch memory errors."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG_RT = "/opt/rocm/lib/llvm/lib/clang"


def _gcc_rt(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _oracle_asan(tmp_path, src_text):
    (tmp_path / "kvq_oracle.c").write_text(src_text)
    shutil.copy(os.path.join(ROOT, "oracle", "kvq_oracle.h"), tmp_path / "kvq_oracle.h")
    so = tmp_path / "oracle_asan.so"
    subprocess.check_call(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-fPIC", "-shared",
                           str(tmp_path / "kvq_oracle.c"), "-o", str(so), "-lm"])
    return so


def _preload(*libs):
    """The sanitizer runtimes first (they must come first), then whatever the
    environment already preloads, unchanged."""
    rest = os.environ.get("LD_PRELOAD", "")
    return " ".join([x for x in libs if x] + ([rest] if rest else []))


def _run_pins(so, files, log=None):
    opts = "detect_leaks=0" + (":log_path=%s" % log if log else "")
    env = dict(os.environ, KVQ_ORACLE_SO=str(so), ASAN_OPTIONS=opts,
               LD_PRELOAD=_preload(_gcc_rt("libasan.so"), _gcc_rt("libubsan.so")))
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] +
                          [os.path.join(ROOT, "tests", f) for f in files],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.mark.skipif(not (_gcc_rt("libasan.so") and _gcc_rt("libubsan.so")), reason="gcc sanitizer runtimes missing")
def test_oracle_pins_under_sanitizers(tmp_path):
    src = open(os.path.join(ROOT, "oracle", "kvq_oracle.c")).read()
    so = _oracle_asan(tmp_path, src)
    r = _run_pins(so, ["test_oracle_pins.py", "test_oracle_key_per_token.py"])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    # control: one byte too few for a flush's codes must be reported
    old = "uint8_t *codes = (uint8_t *)malloc((size_t)G * (size_t)d);"
    assert src.count(old) == 1
    (tmp_path / "bad").mkdir()
    bad = _oracle_asan(tmp_path / "bad", src.replace(old, "uint8_t *codes = (uint8_t *)malloc((size_t)G * (size_t)d - 1);"))
    log = tmp_path / "bad" / "asan"
    r = _run_pins(bad, ["test_oracle_pins.py"], log=log)
    reports = "".join(p.read_text() for p in (tmp_path / "bad").glob("asan*"))
    assert r.returncode != 0 and "heap-buffer-overflow" in reports, r.stdout[-2000:]


def _clang_asan_rt():
    if not os.path.isdir(CLANG_RT):
        return None
    for ver in sorted(os.listdir(CLANG_RT), reverse=True):
        p = os.path.join(CLANG_RT, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


@pytest.mark.skipif(not (os.path.exists(HIPCC) and _clang_asan_rt()), reason="hipcc or its sanitizer runtime missing")
def test_host_runtime_checks_under_sanitizers(tmp_path):
    """The library's host runtime (validation, planning, bookkeeping) built
    with AddressSanitizer and UndefinedBehaviorSanitizer for the host side
    only, linked with the kernels as built; the C ABI's CPU tests pass."""
    sys.path.insert(0, ROOT)
    from decode_attention_streaming_amd import build as bld
    csrc = os.path.join(ROOT, "decode_attention_streaming_amd", "csrc")
    flags = [f for f in bld.FLAGS if not f.startswith("-O")] + ["-O1", "-g"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    # the host runtime is built again, instrumented; the kernels' objects are
    # those of the last build (skip when there is none)
    objs = []
    for src, name, extra in bld.SOURCES:
        if src.endswith(".cpp"):
            obj = str(tmp_path / (name + ".o"))
            subprocess.check_call([HIPCC] + flags + san + extra + ["-c", os.path.join(csrc, src), "-o", obj],
                                  stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        else:
            obj = os.path.join(bld.BUILD, name + ".o")
            if not os.path.exists(obj) or os.path.getmtime(obj) < os.path.getmtime(os.path.join(csrc, src)):
                pytest.skip("kernel objects not built (or older than their sources): run the build first")
        objs.append(obj)
    so = str(tmp_path / "libkvq_asan.so")
    subprocess.check_call([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                           "-Xarch_host", "-fsanitize=undefined", "-o", so] + objs,
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    env = dict(os.environ, KVQ_LIB=so, ASAN_OPTIONS="detect_leaks=0", LD_PRELOAD=_preload(_clang_asan_rt()))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
