"""The host half of the library (page-table lowering, index validation, both
planners, metadata copy) under AddressSanitizer and UndefinedBehaviorSanitizer:
``paged_kv_cache_201_amd/build.py --sanitize`` links host.cpp into the seeded
driver ``tests/host_sanitize.cpp`` (exact-size buffers, random and malformed
page tables, random tunings); any out-of-bounds access, leak or undefined
behaviour aborts it.  CPU only."""
import importlib.util
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("pkv_build", os.path.join(ROOT, "paged_kv_cache_201_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_host_half_under_asan_and_ubsan():
    exe = _build_module().build_host_sanitize()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe, "600"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "host_sanitize ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
