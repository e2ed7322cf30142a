"""The oracle under gcc's AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): a sanitizer build runs the oracle's pins in a child process that
preloads the sanitizer runtimes; any out-of-bounds access, use after free or
undefined behaviour aborts it."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import inspect, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
o = oracle.Oracle({lib!r})
import test_oracle_lmhead, test_oracle_pins, test_oracle_step
ran = 0
for mod in (test_oracle_lmhead, test_oracle_pins, test_oracle_step):
    for name, fn in inspect.getmembers(mod, inspect.isfunction):
        params = inspect.signature(fn).parameters
        if not name.startswith("test_") or any(p not in ("o", "oracle") for p in params):
            continue
        fn(**{{p: o for p in params}})
        ran += 1
print("ran", ran)
"""


def _runtime(name):
    try:
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_oracle_pins_run_clean_under_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not available")
    import oracle
    lib = str(tmp_path / "liboracle_sanitize.so")
    oracle.build(lib, sanitize=True)
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "ran " in r.stdout and int(r.stdout.split("ran ")[-1]) >= 20, r.stdout[-500:]
