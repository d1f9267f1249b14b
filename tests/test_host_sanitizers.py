"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

  * the seeded input generator (fixtures/gen.c) built with gcc and the sanitizers, driven by
    tests/sanitize/fx_driver.c over odd sizes, offsets and encoder edge values;
  * the library's host code (every csrc/*.hip, the sanitizers applied to the host side
    only: device code is built as usual) linked into tests/sanitize/abi_driver.cpp, which
    drives every argument check of the C ABI that fails before any device work, so it runs
    without a GPU.
A sanitizer report makes the driver exit non-zero."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1:detect_leaks=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
pytestmark = pytest.mark.slow


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_fixture_generator_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "fx_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "fixtures", "gen.c"), os.path.join(HERE, "sanitize", "fx_driver.c"),
          "-o", exe, "-lm"])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1"))
    assert "driver ok" in r.stdout


def test_library_host_code_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    csrc = os.path.join(ROOT, "discrete_diffusion_decoding_canvas_amd", "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith(".hip"))
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Wno-unused-result"]
    objs = []
    procs = []
    for src in srcs + [os.path.join(HERE, "sanitize", "abi_driver.cpp")]:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        procs.append((src, subprocess.Popen([HIPCC, *flags, "-c", src, "-o", obj],
                                            stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
        objs.append(obj)
    for src, p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, f"{src}\n{err[-3000:]}"
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, "--offload-arch=gfx950",
          "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", *objs, "-o", exe])
    r = _run([exe], env=ENV)
    assert "driver ok" in r.stdout
