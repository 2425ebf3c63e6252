"""Host sanitizer builds, on the CPU only (nothing here launches a kernel).

* The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
  (abort on the first report) passes its own pin tests.
* libkvrc built with host-side undefined-behaviour traps (signed overflow,
  shifts, bounds, division by zero, null and misaligned accesses) passes the
  C-ABI boundary tests, including sizes at and past every bound: the
  validation arithmetic never overflows.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ORACLE_TESTS = ["tests/test_oracle_rmsnorm.py", "tests/test_oracle_rope.py",
                "tests/test_oracle_quant.py", "tests/test_oracle_fp8.py",
                "tests/test_oracle_scatter.py", "tests/test_oracle_qsa.py",
                "tests/test_oracle_mla.py"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not available")
    return path


def _pytest_with(setup: str, files, env):
    code = (f"import sys; sys.path.insert(0, {ROOT!r}); {setup}; import pytest; "
            f"sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider'] + "
            f"{list(files)!r}))")
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=900)


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    import oracle
    lib = oracle.build(sanitize=True, out=str(tmp_path / "liboracle_kvrc_san.so"))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               LD_PRELOAD=_runtime("libasan.so") + ":" + _runtime("libubsan.so"))
    r = _pytest_with(f"import oracle; oracle._LIB_PATH = {lib!r}", ORACLE_TESTS, env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout


# Host-side undefined-behaviour traps (no runtime library needed); the device
# code is built as usual.
HOST_UB_TRAP_FLAGS = [
    "-Xarch_host", "-fsanitize=signed-integer-overflow,shift,bounds,integer-divide-by-zero,"
    "null,alignment", "-Xarch_host", "-fsanitize-trap=all", "-fno-gpu-sanitize",
]


def test_boundary_under_host_ub_traps(tmp_path):
    from latent_attention_kv_amd import _build
    lib = str(tmp_path / "libkvrc_ubtrap.so")
    srcs = [os.path.join(_build.CSRC, s) for s in _build.SOURCES]
    subprocess.run([_build.hipcc(), *_build.HIPCC_FLAGS, *HOST_UB_TRAP_FLAGS, "-I",
                    _build.INCLUDE, "-I", _build.CSRC, "-o", lib, *srcs], check=True,
                   capture_output=True, timeout=900)
    r = _pytest_with(f"import latent_attention_kv_amd as k; k.LIB_PATH = {lib!r}",
                     ["tests/test_boundary.py"], dict(os.environ))
    # a trap ends the process with SIGILL / SIGTRAP instead of a pytest status
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
