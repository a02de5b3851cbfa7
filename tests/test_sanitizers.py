"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two instrumented builds, each driven by the CPU tests that exercise it, in a
subprocess with the matching sanitizer runtime preloaded:
  - libpa.so with its host code instrumented (hipcc, -fsanitize=address and
    undefined for the host compilation only; device code as usual): the block
    manager's random runs and rule tests (test_kv_manager.py) and the C ABI's
    argument checks (test_abi.py), which return before any launch, and the
    contract checks on host copies (test_validate.py);
  - the C oracle (gcc): its pins (test_oracle.py, test_oracle_rope.py,
    test_oracle_fp8.py) and the input draws (test_workloads.py).
Any sanitizer report ends the subprocess with an error and fails the test.
The builds go to _build/asan/ (ignored by git)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "asan")


def _run(env_extra, tests, log):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = f"detect_leaks=0:log_path={log}"
    env["UBSAN_OPTIONS"] = f"halt_on_error=1:print_stacktrace=1:log_path={log}"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                        *[os.path.join(ROOT, "tests", t) for t in tests]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = [os.path.join(OUT, f) for f in os.listdir(OUT) if f.startswith(os.path.basename(log) + ".")]
    text = "".join(open(p).read() for p in reports)
    assert r.returncode == 0 and not reports, (r.stdout[-3000:] + r.stderr[-3000:] + text[:6000])
    return r.stdout


@pytest.fixture(scope="module")
def outdir():
    os.makedirs(OUT, exist_ok=True)
    for f in os.listdir(OUT):                       # reports of earlier runs
        if f.startswith(("asan_lib.", "asan_oracle.")):
            os.remove(os.path.join(OUT, f))
    return OUT


def test_library_host_code_under_asan_ubsan(outdir):
    from paged_kv_cache_432_amd import _build
    lib = _build.build(out=os.path.join(outdir, "libpa.so"), sanitize=True)
    out = _run({"LD_PRELOAD": _build.asan_runtime(), "PA_LIB": lib}, ["test_kv_manager.py", "test_abi.py", "test_validate.py"],
               os.path.join(outdir, "asan_lib"))
    assert " passed" in out


def test_oracle_under_asan_ubsan(outdir):
    import oracle
    lib = oracle.build_sanitized(os.path.join(outdir, "libpa_oracle.so"))
    rt = " ".join(subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True,
                                 check=True).stdout.strip() for n in ("libasan.so", "libubsan.so"))
    out = _run({"LD_PRELOAD": rt, "PA_ORACLE_LIB": lib},
               ["test_oracle.py", "test_oracle_rope.py", "test_oracle_fp8.py", "test_workloads.py"],
               os.path.join(outdir, "asan_oracle"))
    assert " passed" in out
