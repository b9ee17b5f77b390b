"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only): a sanitized build of oracle/dora_oracle.c runs every
oracle pin in a child process with the ASan runtime preloaded; any
out-of-bounds access, use after free or undefined operation aborts it."""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    if shutil.which("gcc") is None:
        return None
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_asan_runtime() is None, reason="gcc with libasan not available")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import build as OB
    lib = str(tmp_path / "liboracle_sanitized.so")
    OB.build(out=lib, extra=["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                             "-fno-omit-frame-pointer", "-g"])
    script = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})
        from oracle import oracle as O
        O.set_library({lib!r})
        import oracle_pins as P
        names = [n for n in dir(P) if n.startswith("pin_")]
        for n in names:
            getattr(P, n)()
        print("PINS", len(names))
    """)
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    res = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env,
                         timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]
    assert "PINS" in res.stdout and "ERROR: AddressSanitizer" not in res.stderr, res.stderr[-4000:]
    assert "runtime error" not in res.stderr, res.stderr[-4000:]
