"""The library's host code under AddressSanitizer and UndefinedBehaviourSanitizer (CPU only).

Builds libvdit.so with sanitized host code (argument validation, the host plan builder, RoPE
tables, the reuse policy, launch set-up; device code as usual) and runs the host-side ABI
tests (tests/test_abi_host.py: plans bit-exact against the oracle on every workload and on
random rules, every error path) against it in a subprocess that preloads the sanitizer
runtime.  Any report stops that process with a failure."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    from video_diffusion_transformer_rope3d_amd import build
    lib = build.build_sanitized(str(tmp_path / "san"))
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report_load" in nm and "__ubsan_handle" in nm, "host code not instrumented"
    code = (
        "import sys\n"
        f"sys.path[:0] = [{ROOT!r}, {os.path.join(ROOT, 'tests')!r}]\n"
        "import video_diffusion_transformer_rope3d_amd.binding as B\n"
        f"B.LIB_PATH = {lib!r}\n"
        "import pytest\n"
        "rc = pytest.main(['-x', '-q', '-p', 'no:cacheprovider', 'tests/test_abi_host.py'])\n"
        f"assert B._lib is not None and B._lib._name == {lib!r}, 'the sanitized library was not the one loaded'\n"
        "sys.exit(rc)\n")
    env = dict(os.environ, LD_PRELOAD=":".join(p for p in (build.sanitizer_runtime(), os.environ.get("LD_PRELOAD"))
                                                 if p),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1500)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
