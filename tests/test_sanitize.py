"""The host-side validation of every entry point, built once with
AddressSanitizer and UndefinedBehaviorSanitizer (tests/sanitize): every call
with bad arguments is rejected with the documented status before any launch,
and no workspace sizer or check overflows at extreme sizes.  CPU only."""
import os
import shutil

import pytest


def test_host_checks_under_sanitizers(tmp_path):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    from tests.sanitize import build_and_run
    exe = build_and_run.build(str(tmp_path))
    r = build_and_run.run(exe)
    out = r.stdout + r.stderr
    assert "runtime error" not in out, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "host checks: 0 failed" in r.stdout
