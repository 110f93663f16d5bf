"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

* The oracle (oracle/moe_oracle.c) is built with gcc -fsanitize=address,undefined
  and every pin runs against it in a child process that preloads the
  sanitizer runtimes (the Python interpreter itself is not instrumented).  Any
  sanitizer report fails the test.
* Every planted mutant of the oracle is built the same way and must still be
  caught: a pin fails or a sanitizer reports (a mutant that reads past a buffer
  is caught either way).
* The HIP library is rebuilt with the sanitizers on its host code only (each
  -fsanitize directly after -Xarch_host; device code is untouched) and the
  host-side checks of tests/test_abi_cpu.py run against it.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

import oracle.build as ob
from test_oracle_mutants import MUTANTS, SRC

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


ASAN, UBSAN = _runtime("libasan.so"), _runtime("libubsan.so")


def _clang_runtime():
    """The address sanitizer runtime of hipcc's host compiler (clang), which
    also carries the undefined-behaviour handlers."""
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang):
        return None
    p = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                       text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


pytestmark = pytest.mark.skipif(not (ASAN and UBSAN), reason="gcc sanitizer runtimes not found")


def _env():
    env = dict(os.environ)
    env["LD_PRELOAD"] = f"{ASAN}:{UBSAN}"
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "2"
    env["PYTHONPATH"] = os.pathsep.join([ROOT, HERE, env.get("PYTHONPATH", "")])
    return env


PIN_RUNNER = """
import sys, oracle, oracle_pins
orc = oracle.Oracle(sys.argv[1])
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(orc)
    except AssertionError:
        failed.append(pin.__name__)
print("FAILED_PINS", failed, flush=True)
sys.exit(3 if failed else 0)
"""


def _run_pins(lib):
    return subprocess.run([sys.executable, "-c", PIN_RUNNER, lib], capture_output=True, text=True,
                          env=_env(), timeout=600)


def _sanitizer_report(text):
    return "ERROR: AddressSanitizer" in text or "runtime error:" in text


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = ob.build(out=str(tmp_path / "liboracle_san.so"), extra=SAN)
    r = _run_pins(lib)
    assert not _sanitizer_report(r.stderr), r.stderr[-4000:]
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-2000:])
    assert "FAILED_PINS []" in r.stdout


def test_oracle_mutants_caught_under_sanitizers(tmp_path):
    with open(SRC) as f:
        text = f.read()

    def one(name):
        old, new = MUTANTS[name]
        d = tmp_path / name
        d.mkdir()
        src = d / "mut.c"
        src.write_text(text.replace(old, new))
        lib = ob.build(src=str(src), out=str(d / "libmut.so"), extra=SAN)
        r = _run_pins(lib)
        caught = r.returncode != 0 and ("FAILED_PINS [" in r.stdout and "FAILED_PINS []" not in r.stdout
                                        or _sanitizer_report(r.stderr))
        return name, caught, r.returncode

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(one, sorted(MUTANTS)))
    missed = [(n, rc) for n, caught, rc in results if not caught]
    assert not missed, f"mutants not caught under the sanitizers: {missed}"


def test_library_host_code_under_sanitizers(tmp_path):
    from bit_routed_expert_moe_amd import build as pb
    lib = str(tmp_path / "libmoe_layer.so")
    pb.build(extra=["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-omit-frame-pointer"], out=lib)
    crt = _clang_runtime()
    if crt is None:
        pytest.skip("clang's sanitizer runtime not found")
    env = _env()
    env["LD_PRELOAD"] = crt
    env["MOE_LAYER_LIB"] = lib
    probe = subprocess.run([sys.executable, "-c", "from bit_routed_expert_moe_amd import layer as L; "
                            "L.lib(); print(L.LIB_PATH)"], capture_output=True, text=True, env=env,
                           timeout=300, cwd=ROOT)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi_cpu.py")], capture_output=True, text=True, env=env,
                       timeout=600, cwd=ROOT)
    assert not _sanitizer_report(r.stdout + r.stderr), (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
