"""Host checks of the benchmark's algorithmic byte counts against the per-query figures
derived from the storage formats: an MXFP4 index key is d_i/2 data bytes plus d_i/32 scale
bytes (68 B at d_i=128), an entry is 448 FP8 bytes, 64 bf16 RoPE dims and a 4-byte scale
(580 B at d=512), and the decode query is 64 heads x 512 bf16 in, fp32 out."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_index_bytes_per_query_at_1m():
    # 262,144 keys x 68 B + 8 heads x (68 B of query + 4 B of head weight)
    assert bench.index_bytes_per_query(262144, 8, 128) == 262144 * 68 + 8 * 72 == 17826368


def test_step_bytes_per_query_at_1m_and_64k():
    entry = 448 + 64 * 2 + 4
    q_out = 64 * 512 * 2 + 64 * 512 * 4
    assert bench.step_bytes_per_query(262144, 8, 128, 1024, 128, 64, 512) == \
        262144 * 68 + 8 * 72 + (1024 + 128) * entry + q_out == 18691136
    # the 64K-context decode: 16,384 keys per query
    assert bench.step_bytes_per_query(16384, 8, 128, 1024, 128, 64, 512) == \
        16384 * 68 + 8 * 72 + (1024 + 128) * entry + q_out


def test_index_excess_bytes():
    # the fp32 score row and one 4-byte summary key per 32 columns
    assert bench.index_excess_bytes_per_query(262144) == 262144 * 4 + 8192 * 4
    assert bench.index_excess_bytes_per_query(33) == 33 * 4 + 2 * 4


def test_more_than_one_gpu_is_refused():
    # the benchmark measures one GPU; asking for more exits with a message and status 2 before
    # anything touches a device
    import subprocess

    for argv, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                           timeout=300, env=dict(os.environ, **env))
        assert r.returncode == 2
        assert "one GPU" in r.stderr and r.stdout == ""
