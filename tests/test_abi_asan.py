"""AddressSanitizer and UndefinedBehaviorSanitizer pass over the host side of the C ABI (no GPU needed).

The library's sources are compiled for gfx950 with the sanitizer applied to the
host pass only, linked with ``tests/asan/abi_host_driver.cpp`` and run: the driver
exercises status strings, configuration and argument validation, workspace
sizing and every rejection path of the forward entry points, all of which return
before the first HIP call.  The sanitizers turn any out-of-bounds access, use
after free, leak or undefined behaviour (signed overflow, misaligned access,
bad shift, ...) on those paths into a failure.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
CSRC = ROOT / "sparse_expert_gemv_amd" / "csrc"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# The sanitizers are applied to the host compilation only.
SAN = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer"]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"{' '.join(map(str, cmd))}\n{r.stderr[-4000:]}"


@pytest.mark.skipif(not Path(HIPCC).exists(), reason="hipcc not installed")
def test_abi_host_paths_under_asan(tmp_path):
    sources = sorted(CSRC.glob("*.hip"))
    assert sources, "no HIP sources found"
    common = ["-std=c++17", "-O1", "-g", "-fPIC", f"-I{ROOT / 'include'}", f"-I{CSRC}"] + SAN
    jobs = [[HIPCC, "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", *common, "-c", str(s), "-o", str(tmp_path / (s.stem + ".o"))]
            for s in sources]
    jobs.append([HIPCC, *common, "-c", str(ROOT / "tests" / "asan" / "abi_host_driver.cpp"),
                 "-o", str(tmp_path / "driver.o")])
    with ThreadPoolExecutor(max_workers=min(len(jobs), 6)) as pool:
        list(pool.map(lambda c: _run(c, tmp_path), jobs))
    objs = [str(tmp_path / (s.stem + ".o")) for s in sources] + [str(tmp_path / "driver.o")]
    exe = tmp_path / "abi_driver"
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address,undefined", *objs,
          "-o", str(exe)], tmp_path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe)], cwd=tmp_path, env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, f"rc={r.returncode}\n{r.stdout}\n{r.stderr[-6000:]}"
    assert "all checks passed" in r.stdout
