"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only):
the fp64 oracle (gcc build, gcc's runtime preloaded) runs its pin tests, and
the C ABI's host code (hipcc build with the sanitizers on the host side only,
clang's runtime preloaded) runs the validation and export tests. Every
finding aborts the child run (no recovery), so a clean exit means none."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ORACLE_TESTS = ["tests/test_oracle_plan.py", "tests/test_oracle_attn.py",
                "tests/test_oracle_locality.py", "tests/test_oracle_validate.py",
                "tests/test_oracle_rescale.py", "tests/test_oracle_baseline.py",
                "tests/test_oracle_fullmask.py", "tests/test_oracle_layer.py"]
ABI_TESTS = ["tests/test_abi_validation.py", "tests/test_abi.py"]


def run_child(tests, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider"] +
                       tests, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
    return r


def imports(lib, prefix):
    out = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    return any(prefix in line for line in out.splitlines())


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    import oracle
    lib = oracle.build(sanitize_to=str(tmp_path / "liboracle_san.so"))
    assert imports(lib, "__asan_report") and imports(lib, "__ubsan_handle")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    run_child(ORACLE_TESTS, {"LD_PRELOAD": asan, "SPLITKV_ORACLE_LIB": lib})


def test_abi_host_code_under_address_and_ub_sanitizers(tmp_path):
    from block_sparse_cross_amd import build
    lib = build.build(host_sanitize_to=str(tmp_path / "libsplitkv_san.so"))
    assert imports(lib, "__asan_report") and imports(lib, "__ubsan_handle")
    run_child(ABI_TESTS, {"LD_PRELOAD": build.host_asan_runtime(), "SPLITKV_LIB": lib})
