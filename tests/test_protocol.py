"""CPU model of the fused schedule's copy protocol (tests/protocol_model.cpp), built with g++ from
the library's own chunk / piece map and tile walk (allgather_gemm_amd/csrc/ag_protocol.hpp).

Workgroups run as threads under the kernel's rules (waiters copy whole pieces, running waves copy
one slice per K step, everyone drains the counters before exiting).  The model checks that every
piece is copied exactly once, that no flag rises before all of its chunk's bytes have landed, that
every tile finds its rows in place, that the gathered buffer ends equal to the concatenation of the
shards, and that no wait outlives a deadline (deadlock).  Shapes: the workloads' shard, chunk and
tile geometry (K reduced, which only changes the piece count), ragged ones, and every local shard.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("protocol") / "protocol_model")
    subprocess.run(["g++", "-std=c++17", "-O2", "-pthread", "-Wall", "-I",
                    os.path.join(ROOT, "allgather_gemm_amd", "csrc"),
                    os.path.join(ROOT, "tests", "protocol_model.cpp"), "-o", exe], check=True)
    return exe


def run_model(exe, N, H, K, cb, local, grid, Nc, trickle=1, piece=16384, slice_=1024, seed=1):
    args = [str(x) for x in (N, H, K, cb, local, grid, 256, 256, Nc, trickle, piece, slice_, seed)]
    res = subprocess.run([exe] + args, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.startswith("OK"), (args, res.stdout, res.stderr)
    return res.stdout


@pytest.mark.parametrize("N,H,K,cb,Nc,grid", [
    (8, 1024, 256, 128, 2048, 256),    # square workload geometry (K reduced)
    (8, 2048, 128, 256, 2048, 256),    # MLP-up geometry
    (8, 500, 256, 100, 2048, 256),     # ragged: tiles straddle shards, edge chunks of the local shard
    (4, 64, 128, 32, 128, 4),          # tiny workload
])
@pytest.mark.parametrize("trickle", [0, 1])
def test_workload_geometries(model, N, H, K, cb, Nc, grid, trickle):
    for local in sorted({0, 1, N // 2, N - 1}):
        run_model(model, N, H, K, cb, local, grid, Nc, trickle=trickle, seed=local + 1)


@pytest.mark.parametrize("N,H,K,cb,local,grid,Nc,piece,slice_", [
    (3, 100, 200, 7, 1, 16, 300, 2048, 1024),       # chunks of 7 rows, pieces smaller than a chunk
    (1, 300, 40, 33, 0, 8, 260, 16384, 1024),       # one shard: nothing is waited for, all drained
    (8, 50, 64, 10, 5, 32, 300, 1024, 1024),        # every tile straddles shards
    (5, 200, 136, 64, 4, 24, 514, 3072, 1024),      # short last chunk of every shard
    (8, 640, 512, 160, 5, 64, 5120, 16384, 1024),   # more tiles than workgroups
    (2, 513, 8, 1, 1, 12, 700, 16, 16),             # one-row chunks, 16-byte pieces
    (7, 97, 24, 97, 6, 5, 40, 4096, 1024),          # one chunk per shard, H not a tile multiple
])
def test_ragged_and_degenerate_geometries(model, N, H, K, cb, local, grid, Nc, piece, slice_):
    for seed in (1, 2, 3):
        run_model(model, N, H, K, cb, local, grid, Nc, piece=piece, slice_=slice_, seed=seed)
