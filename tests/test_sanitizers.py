"""Host code under the sanitizers (CPU only).

* The CPU oracle (oracle/oracle.c), every function driven on small ragged inputs by
  tests/oracle_sanitize.c, built with AddressSanitizer and UndefinedBehaviorSanitizer.
* The copy protocol's model (tests/protocol_model.cpp, which includes the library's own
  ag_protocol.hpp chunk/piece map and tile walk), built once with AddressSanitizer +
  UndefinedBehaviorSanitizer and once with ThreadSanitizer: its workgroups are threads that claim,
  copy and publish pieces through atomics, so a data race in the protocol's host-side model shows
  up here.
Both use gcc/g++ only; no GPU code is built with a sanitizer.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="gcc/g++ not installed")


def _run(exe, args=(), env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    res = subprocess.run([exe] + [str(a) for a in args], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0 and res.stdout.startswith("OK"), (args, res.stdout[-2000:], res.stderr[-4000:])


def test_oracle_under_address_and_undefined_behavior_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN, "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "tests", "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "oracle.c"),
                    "-lm", "-o", exe], check=True)
    _run(exe, env_extra={"OMP_NUM_THREADS": "4"})


PROTOCOL_CASES = [
    # N, H, K, cb, local, grid, bm, bn, Nc, trickle, piece, slice, seed
    (8, 500, 256, 100, 3, 256, 256, 256, 2048, 1, 16384, 1024, 1),   # ragged workload geometry
    (3, 100, 200, 7, 1, 16, 256, 256, 300, 1, 2048, 1024, 2),        # pieces smaller than a chunk
    (2, 513, 8, 1, 1, 12, 256, 256, 700, 1, 16, 16, 3),              # one-row chunks, 16-byte pieces
    (7, 97, 24, 97, 6, 5, 256, 256, 40, 0, 4096, 1024, 1),           # one chunk per shard
]


@pytest.mark.parametrize("flags,tag", [(SAN, "asan"), (["-fsanitize=thread", "-g", "-O1"], "tsan")])
def test_protocol_model_under_sanitizers(tmp_path, flags, tag):
    exe = str(tmp_path / ("protocol_model_" + tag))
    subprocess.run(["g++", "-std=c++17", "-pthread", *flags, "-I", os.path.join(ROOT, "allgather_gemm_amd", "csrc"),
                    os.path.join(ROOT, "tests", "protocol_model.cpp"), "-o", exe], check=True)
    for case in PROTOCOL_CASES:
        _run(exe, case)
