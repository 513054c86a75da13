"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code only) runs every pin in a child process: an out-of-bounds access,
use after free, signed overflow, misaligned load or other undefined behaviour
anywhere the pins reach aborts the child and fails the test (CPU only)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

RUNNER = r"""
import json, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
from oracle_pins import ALL_PINS
lib = oracle.load({lib!r})
res = {{}}
for pin in ALL_PINS:
    pin(lib)
    res[pin.__name__] = "pass"
print(json.dumps(res))
"""


def _runtime(name):
    p = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_pins_pass_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    import oracle
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle.build(extra_flags=("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                    "-fno-omit-frame-pointer", "-g"),
                       out_path=str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["OMP_NUM_THREADS"] = "4"
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=900, env=env)
    assert p.returncode == 0, "sanitized oracle failed:\n" + p.stderr[-4000:]
    res = json.loads(p.stdout.strip().splitlines()[-1])
    from oracle_pins import ALL_PINS
    assert set(res) == {pin.__name__ for pin in ALL_PINS}


def test_sanitizer_catches_a_planted_overflow(tmp_path):
    """The same harness on a copy of the oracle with a one-past-the-end write
    in the selection: the child must abort."""
    import oracle
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    src = open(os.path.join(ROOT, "oracle", "vq_oracle.c")).read()
    old = "    for (long long e = 0; e < total; ++e) keep[e] = 1;"
    assert src.count(old) == 1
    msrc = tmp_path / "planted.c"
    msrc.write_text(src.replace(old, "    for (long long e = 0; e <= total; ++e) keep[e] = 1;"))
    lib = oracle.build(extra_flags=("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                    "-fno-omit-frame-pointer", "-g"),
                       out_path=str(tmp_path / "libplanted.so"), src=str(msrc))
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["OMP_NUM_THREADS"] = "4"
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=900, env=env)
    assert p.returncode != 0 and "AddressSanitizer" in p.stderr
