"""The C ABI's host code (argument validation, workspace sizing, the entry
points' error paths) under AddressSanitizer and UndefinedBehaviorSanitizer:
the host part of prism_api.hip is built with both, and tests/test_abi_host.py
runs against that build in a child process (the sanitizer runtime preloaded
into it), failing on any report."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_host_checks_under_asan_and_ubsan(tmp_path):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a preload is already set for this process tree; it is left as it is")
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("host-only check: runs where no GPU is visible")
    from token_sparse_attention_gqa_amd import build
    lib = build.build_host_sanitized()
    logs = tmp_path / "san"
    env = dict(os.environ)
    env.update({
        "PRISM_LIBRARY": lib,
        "LD_PRELOAD": build.asan_runtime(),
        # the interpreter and the libraries it loads are not instrumented:
        # leak reports and cross-library checks would be about them
        "ASAN_OPTIONS": f"detect_leaks=0:detect_odr_violation=0:alloc_dealloc_mismatch=0:"
                        f"abort_on_error=1:log_path={logs}",
        "UBSAN_OPTIONS": f"halt_on_error=1:print_stacktrace=1:log_path={logs}",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = sorted(p for p in tmp_path.iterdir() if p.name.startswith("san"))
    text = "".join(p.read_text()[:4000] for p in reports)
    assert not reports, f"sanitizer reports:\n{text}"
    assert r.returncode == 0, f"test_abi_host.py failed under the sanitizers:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    assert " passed" in r.stdout
