"""The C ABI's host-side code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The library is rebuilt from the same sources with the sanitizers on its host code only (each
-fsanitize= flag after -Xarch_host; the device code is compiled as in the product build) into a
temporary directory. A child interpreter then runs the host tests of test_capi_host.py against
that build, with the ASan runtime preloaded. Those tests cover the exports, moe_strerror,
moe_mpad_max and every argument check, and the checks return before any GPU work. A sanitizer
report, or a check returning another status than the documented one, fails the test.
"""
import os
import subprocess
import sys

import pytest

from mxfp4_mixture_experts_route_amd import build as moe_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# host code only: each flag directly after -Xarch_host
SAN = ("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
       "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer").split()


def asan_runtime() -> str:
    r = subprocess.run([moe_build.hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else ""


@pytest.mark.timeout(900)
def test_host_argument_checks_clean_under_asan_and_ubsan(tmp_path):
    rt = asan_runtime()
    if not rt:
        pytest.skip("no AddressSanitizer runtime next to hipcc")
    so = moe_build.build(extra=SAN, out_path=str(tmp_path / "libmoe_mx4_san.so"),
                         build_dir=str(tmp_path / "obj"), link_extra=SAN)
    env = dict(os.environ)
    env.update(MOE_MX4_LIB=so, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child maps the sanitized build and the ASan runtime (not the in-tree library)
    probe = ("import sys; sys.path.insert(0, %r)\n"
             "from mxfp4_mixture_experts_route_amd import _lib\n"
             "L = _lib.lib()\n"
             "maps = open('/proc/self/maps').read()\n"
             "assert %r in maps, 'sanitized build not mapped'\n"
             "assert 'libclang_rt.asan' in maps, 'ASan runtime not mapped'\n"
             "assert 'libmoe_mx4.so' not in maps.replace('libmoe_mx4_san.so', '')\n"
             "print('ok')\n") % (ROOT, so)
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and "ok" in r.stdout, (r.stdout + r.stderr)[-3000:]
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_capi_host.py"), "-q",
           "-p", "no:cacheprovider", "-m", "not gpu",
           "-k", "not binds_to_torchs_hip_runtime"]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
