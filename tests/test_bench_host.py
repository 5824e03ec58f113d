"""Host checks of bench.py: its roofline ledgers against the figures derived
from the chunkwise form (per token-head at C = 64, d = 128: 1 540 algorithmic
bytes and 140 629 useful flops for the forward; one decode step over 256
sequences x 32 heads moves 1 086 357 504 bytes), and the one-GPU guard.
No GPU is touched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_forward_byte_ledger():
    # q, k, v, o in bf16 (4 x 256 B), alpha fp32 (512 B), beta fp32 (4 B)
    assert bench.FWD_BYTES_PER_TOKEN_HEAD == 1540
    # the 64K-token, 32-head workload with S_0 read and S_T written (fp32)
    units = 1 * 32 * 65536
    assert bench.FWD_BYTES_PER_TOKEN_HEAD * units + 2 * 32 * 128 * 128 * 4 == 3_233_808_384


def test_forward_flop_ledger():
    # 6 d^2 for U' = U - W S, S <- gamma S + Kt^T U', Qh S; C d_k (A), C (d_k + d_v)
    # (T X), C d_k (Qh Kb^T), C d_v (P U'), C^2 / 3 (the substitution)
    assert bench.fwd_flops_per_token_head(64, 128, 128) == 140_629
    assert bench.FWD_FLOPS_PER_TOKEN_HEAD == 140_629
    # arithmetic intensity ~91 flop per algorithmic byte: far below the bf16 ridge
    assert 90 < 140_629 / 1540 < 92


def test_decode_byte_ledger():
    assert bench.decode_bytes_per_step(256, 32, 128, 128) == 1_086_357_504
    # the other gate forms change only the gate's bytes
    n = 256 * 32
    assert (bench.decode_bytes_per_step(256, 32, 128, 128, "alpha")
            - bench.decode_bytes_per_step(256, 32, 128, 128, "softplus")) == n * 128 * 2
    assert (bench.decode_bytes_per_step(256, 32, 128, 128, "alpha")
            - bench.decode_bytes_per_step(256, 32, 128, 128, "scalar")) == n * (128 * 4 - 4)


def test_backward_mixed_roofline():
    f16, f32 = bench.bwd_flops_split(64, 128, 128)
    assert f16 + f32 == bench.bwd_flops_per_token_head(64, 128, 128)
    assert abs((f16 + f32) - 410_966) < 1      # 2 (8 dk dv + 5.5 C dk + 3 C dv + 7/6 C^2)
    peak = bench.bwd_mixed_peak(64, 128, 128)
    # between the fp32 and the fp16 matrix-core peaks, pulled towards fp32
    assert bench.FP32_MFMA_PEAK_TFLOPS < peak < bench.BF16_MFMA_PEAK_TFLOPS
    assert abs(peak - 509.3) < 0.5


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                       ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       env={**os.environ, **env}, capture_output=True, text=True, timeout=60)
    assert r.returncode != 0
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""
