"""The binding has no non-HIP path: a missing or out-of-date library must raise.

Runs on the CPU: loading a shared library makes no GPU call. Each case runs in
a child process so that the package's cached handle is untouched.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load_with(path: str) -> subprocess.CompletedProcess:
    code = (
        "import mixture_experts_lora_amd._lib as L\n"
        f"L.LIB_PATH = {path!r}\n"
        "L._lib = None\n"
        "try:\n"
        "    L.load()\n"
        "except RuntimeError as e:\n"
        "    print('RAISED', e)\n"
        "else:\n"
        "    print('LOADED')\n"
    )
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                          timeout=120)


def test_missing_library_raises():
    r = _load_with(os.path.join(ROOT, "mixture_experts_lora_amd", "no_such_library.so"))
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("RAISED"), r.stdout
    assert "is missing" in r.stdout


def test_library_without_the_exports_raises():
    # any real shared object lacking the C ABI stands for an out-of-date build:
    # this process's own libc, by the absolute path it was mapped from
    with open("/proc/self/maps") as f:
        libc = next(ln.split()[-1] for ln in f if "/libc.so" in ln or "/libc-" in ln)
    assert os.path.isabs(libc) and os.path.exists(libc)
    r = _load_with(libc)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("RAISED"), r.stdout
    assert "lacks moe_" in r.stdout
