"""CPU sanitizer runs (no GPU): the oracle and the library's host code built
with AddressSanitizer + UndefinedBehaviorSanitizer, each exercised by the CPU
tests that drive it, in a child process with the matching runtime preloaded.
Any sanitizer report aborts the child (-fno-sanitize-recover), so a clean exit
status with no report in its output is the pass condition."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _run_child(args, env_extra, timeout):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"  # the interpreter itself keeps its arenas
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.setdefault("OMP_NUM_THREADS", "4")
    # -s: a sanitizer report goes to the child's own stderr, not into pytest's capture
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider", *args],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for rep in REPORTS:
        assert rep not in out, out[-4000:]
    return out


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    import oracle

    lib = oracle.build_sanitized(str(tmp_path / "liboracle_asan.so"))
    gcc_rt = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True).stdout.strip()
              for n in ("libasan.so", "libubsan.so")]
    # every oracle function on small inputs: decode, rows, pooled forward,
    # grouping, grouped forward, backward, K-core forward / backward, SGD
    sel = ("not multilinear and not digests and not reproducible_and_shaped and not [4-32] "
           "and not three_core_oracle and not selected_slices and not [4-64]")
    out = _run_child([os.path.join("tests", "test_oracle_pins.py"), "-k", sel],
                     {"TT_ORACLE_LIB": lib, "LD_PRELOAD": ":".join(gcc_rt)}, timeout=900)
    assert " passed" in out


def test_library_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    from tensor_train_compressed_gather_amd import build as hipbuild

    try:
        rt = hipbuild.asan_runtime()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    lib = hipbuild.build_host_sanitized(str(tmp_path / "libtt_emb_asan.so"))
    # argument checks of every entry point, create-time shape checks, the
    # victim order, status strings and the binding's own checks
    out = _run_child([os.path.join("tests", "test_abi.py")], {"TT_EMB_LIB": lib, "LD_PRELOAD": rt}, timeout=600)
    assert " passed" in out
