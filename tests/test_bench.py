"""CPU checks of the bench's accounting: the algorithmic work and bytes it
divides by, pinned to figures derived by hand from the problem definition,
the comment-insensitive hash that ties stored HBM counters to the score
kernel's code, and the refusal of a multi-GPU run."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L, N, H, D, K = 1 << 20, 8192, 64, 128, 2048


def test_scoring_flops_count_every_causal_pair():
    # queries at L - n .. L - 1 see t + 1 keys: n L - n (n - 1) / 2 pairs
    pairs = N * L - N * (N - 1) // 2
    assert pairs == 8_556_384_256
    assert bench.scoring_flops(L, N, H, D, L - N) == 2.0 * H * D * pairs
    assert abs(bench.scoring_flops(L, N, H, D, L - N) - 1.4019e14) < 1e10


def test_replay_bytes_per_format():
    # per entry: key row + index + output score; per query: its rows and weights
    assert bench.replay_bytes(N, H, D, K, "bf16") == N * K * (2 * D + 8) + N * H * (2 * D + 4)
    assert bench.replay_bytes(N, H, D, K, "bf16") == 4_565_499_904
    # FP8 adds the per-token scales of every key row and of the query
    assert bench.replay_bytes(N, H, D, K, "fp8") == N * K * (D + 4 + 8) + N * (H * (D + 4) + 4)
    assert bench.replay_bytes(N, H, D, K, "fp8") == 2_418_049_024
    # MX rows carry one scale byte per 32 elements
    assert bench.replay_bytes(N, H, D, K, "mxfp4") == N * K * (D // 2 + 4 + 8) + N * H * (D // 2 + 4 + 4)


def test_backward_bytes():
    # per entry key row, index, dI; per query q, w read and dq, dw written; dk once
    bf = bench.backward_bytes(L, N, H, D, K)
    assert bf == N * K * (2 * D + 8) + N * (H * (2 * D + 4) + H * (4 * D + 4)) + L * D * 4
    assert bf == 5_372_903_424
    assert bench.backward_bytes(L, N, H, D, K, "fp8") < bf


def test_kernel_hash_ignores_comments_and_spacing(tmp_path):
    ref = bench.kernel_hash()
    for rel in bench.KERNEL_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    old_root = bench.ROOT
    try:
        bench.ROOT = str(tmp_path)
        assert bench.kernel_hash() == ref
        first = tmp_path / bench.KERNEL_SOURCES[0]
        first.write_text("// an added line comment\n/* and a\n block one */\n\n" + first.read_text())
        assert bench.kernel_hash() == ref
        first.write_text(first.read_text().replace("constexpr int kTK = 64;", "constexpr int kTK = 32;"))
        assert bench.kernel_hash() != ref
    finally:
        bench.ROOT = old_root


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""
