"""CPU sanitizer tier: the oracle and the library's host code built with
AddressSanitizer and UndefinedBehaviorSanitizer, then the CPU pins of the
oracle and the C-ABI argument checks run against those builds in child
processes (the ASan runtime has to be loaded first, so it is preloaded
there).  Any report aborts the child and fails the test.

The library's device code is the ordinary build (its objects are reused);
only the host side -- argument validation, workspace plans, launch set-up --
is instrumented, which is where a host-side bounds or overflow mistake would
live.  No GPU is touched: every ABI test returns before anything launches."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sparse_attention_kv_paged_amd")
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:detect_odr_violation=0:abort_on_error=1:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run_child(code, preload, extra_env=None, timeout=900):
    env = dict(os.environ, **ENV_SAN, LD_PRELOAD=preload, PYTHONPATH=ROOT, OMP_NUM_THREADS="4")
    env.update(extra_env or {})
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    out = r.stdout[-4000:] + "\n" + r.stderr[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out
    assert r.returncode == 0, out
    return out


def test_oracle_pins_under_asan_and_ubsan():
    """Every oracle pin (tests/test_oracle_pins.py) against the sanitized oracle."""
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("gcc's ASan runtime is not installed")
    with tempfile.TemporaryDirectory() as tmp:
        so = os.path.join(tmp, "liboracle_san.so")
        subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-shared", "-fPIC", *SAN,
                        os.path.join(ROOT, "oracle", "idx_oracle.c"), "-o", so, "-lm"], check=True)
        code = ("import sys, pytest\n"
                "from oracle import oracle\n"
                f"oracle._LIB = {so!r}\n"
                "oracle._lib = None\n"
                "sys.exit(pytest.main(['-q', '-s', '-x', '-p', 'no:cacheprovider', 'tests/test_oracle_pins.py']))\n")
        out = _run_child(code, libasan)
        assert " passed" in out, out


def test_abi_checks_under_asan_and_ubsan():
    """The C-ABI tests (tests/test_abi.py) against libidx.so whose host code
    is sanitized."""
    objs = [os.path.join(ROOT, "_build", f + ".o") for f in ("idx_score.hip", "idx_topk.hip", "idx_write.hip",
                                                             "idx_level1.hip")]
    if not all(os.path.exists(o) for o in objs) or not os.path.exists(HIPCC):
        pytest.skip("the library is not built here")
    rt = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        pytest.skip("clang's ASan runtime is not installed")
    host_san = [x for f in SAN for x in ("-Xarch_host", f)]
    with tempfile.TemporaryDirectory() as tmp:
        api_o = os.path.join(tmp, "idx_api.o")
        subprocess.run([HIPCC, "-xhip", "-O1", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                        "-I", os.path.join(ROOT, "include"), *host_san, "-c",
                        os.path.join(PKG, "csrc", "idx_api.cpp"), "-o", api_o], check=True,
                       capture_output=True)
        so = os.path.join(tmp, "libidx_san.so")
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address,undefined",
                        "-shared-libsan", api_o, *objs, "-o", so], check=True, capture_output=True)
        code = ("import sys, pytest\n"
                "from sparse_attention_kv_paged_amd import lib as L\n"
                f"L._lib = L.load({so!r})\n"
                "sys.exit(pytest.main(['-q', '-s', '-x', '-p', 'no:cacheprovider', 'tests/test_abi.py']))\n")
        out = _run_child(code, rt)
        assert " passed" in out, out


def test_sanitizers_are_active():
    """The tier would pass vacuously if the instrumentation were missing: a
    copy of the oracle with one planted out-of-bounds write (the per-key
    buffer one element short) must be reported by the same pin run, and the
    sanitized library must call into the ASan runtime."""
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(libasan) or not os.path.exists(libasan):
        pytest.skip("gcc's ASan runtime is not installed")
    src = open(os.path.join(ROOT, "oracle", "idx_oracle.c")).read()
    anchor = "double *k = (double *)malloc(sizeof(double) * (size_t)D);"
    assert src.count(anchor) >= 1
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "planted.c")
        with open(path, "w") as f:
            f.write(src.replace(anchor, "double *k = (double *)malloc(sizeof(double) * (size_t)(D - 1));"))
        so = os.path.join(tmp, "liboracle_planted.so")
        subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-shared", "-fPIC", *SAN, path, "-o", so, "-lm"],
                       check=True)
        code = ("import sys, pytest\n"
                "from oracle import oracle\n"
                f"oracle._LIB = {so!r}\n"
                "oracle._lib = None\n"
                "sys.exit(pytest.main(['-q', '-s', '-x', '-p', 'no:cacheprovider', 'tests/test_oracle_pins.py',"
                " '-k', 'one_hot']))\n")
        env = dict(os.environ, **ENV_SAN, LD_PRELOAD=libasan, PYTHONPATH=ROOT, OMP_NUM_THREADS="2")
        r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=600)
        assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]
    objs = [os.path.join(ROOT, "_build", f + ".o") for f in ("idx_score.hip", "idx_topk.hip")]
    if all(os.path.exists(o) for o in objs) and os.path.exists(HIPCC):
        with tempfile.TemporaryDirectory() as tmp:
            api_o = os.path.join(tmp, "idx_api.o")
            subprocess.run([HIPCC, "-xhip", "-O1", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
                            "-I", os.path.join(ROOT, "include"), *[x for f in SAN for x in ("-Xarch_host", f)],
                            "-c", os.path.join(PKG, "csrc", "idx_api.cpp"), "-o", api_o], check=True,
                           capture_output=True)
            syms = subprocess.run(["nm", "-u", api_o], capture_output=True, text=True).stdout
            assert "__asan_" in syms and "__ubsan_" in syms
