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


# ---------------------------------------------------------------------------
# The profiles/ summaries: bench.py --summarize on small rocprofv3-shaped CSVs
# ---------------------------------------------------------------------------
PREP = "void kda::(anonymous namespace)::prep_kernel<128, 128, true, 0>(kda::(anonymous namespace)::PrepParams)"
STATE = ("void kda::(anonymous namespace)::state_split_kernel<128, 128, true>"
         "(kda::(anonymous namespace)::StateParams)")
OTHER = "void at::native::elementwise_kernel<128, 4>(int)"
COPY = "void bench_copy_kernel(float const*, float*)"


def _write_csv(path, header, rows):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)
    return str(path)


def test_trace_summary_keeps_library_kernels_and_sums_the_forward(tmp_path, capsys):
    p = _write_csv(tmp_path / "run_kernel_stats.csv",
                   ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
                   [[PREP, 4, 4_400_000, 1_100_000, 50, 1_000_000, 1_200_000, 0],
                    [STATE, 4, 4_000_000, 1_000_000, 40, 990_000, 1_010_000, 0],
                    [OTHER, 9, 900_000, 100_000, 10, 1, 2, 0]])
    bench.summarize("trace", [p], "t", ["cmd"])
    out = capsys.readouterr().out
    assert "prep_kernel<128, 128, true, 0>" in out and "state_split_kernel<128, 128, true>" in out
    assert "elementwise" not in out
    assert "forward kernels, sum of averages: 2100.00 us" in out


def test_trace_summary_sums_the_generic_path_per_chunk_size(tmp_path, capsys):
    ns = "void kda::(anonymous namespace)::"
    rows = [[ns + "gprep_kernel<128, 128, 32, true, 0>(kda::(anonymous namespace)::GParams)", 2, 4_000_000, 2_000_000, 0, 1, 2, 0],
            [ns + "gchain_kernel<128, 128, 32>(kda::(anonymous namespace)::GParams)", 2, 6_000_000, 3_000_000, 0, 1, 2, 0],
            [ns + "gout_kernel<128, 128, 128, true>(kda::(anonymous namespace)::GParams)", 2, 3_000_000, 1_500_000, 0, 1, 2, 0],
            [PREP, 4, 4_400_000, 1_100_000, 50, 1_000_000, 1_200_000, 0]]
    p = _write_csv(tmp_path / "run_kernel_stats.csv",
                   ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"], rows)
    bench.summarize("trace", [p], "t", [], kernels=["gprep_kernel", "gchain_kernel", "gout_kernel"])
    out = capsys.readouterr().out
    assert "prep_kernel<128, 128, true, 0>" not in out          # filtered out by --kernels
    assert "chunk-32 forward (generic path) kernels (plan_kernel not included), sum of averages: 5000.00 us" in out
    assert "chunk-128 forward (generic path) kernels (plan_kernel not included), sum of averages: 1500.00 us" in out


def test_traffic_summary_scales_by_the_copy(tmp_path, capsys):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    f = _write_csv(tmp_path / "f.csv", hdr, [[PREP, "FETCH_SIZE", 1000], [PREP, "FETCH_SIZE", 3000]])
    w = _write_csv(tmp_path / "w.csv", hdr, [[PREP, "WRITE_SIZE", 500]])
    # the 1 GiB copy reads as 0.5 GiB of FETCH_SIZE and 1 GiB of WRITE_SIZE
    cf = _write_csv(tmp_path / "cf.csv", hdr, [[COPY, "FETCH_SIZE", (1 << 30) / 2 / 1024]])
    cw = _write_csv(tmp_path / "cw.csv", hdr, [[COPY, "WRITE_SIZE", (1 << 30) / 1024]])
    bench.summarize("traffic", [f, w, cf, cw], "t", [])
    out = capsys.readouterr().out
    assert "fetch_scale: 2.000000" in out and "write_scale: 1.000000" in out
    # mean FETCH_SIZE 2000 KiB x 2, WRITE_SIZE 500 KiB x 1
    assert f"read_bytes {2000 * 1024 * 2} write_bytes {500 * 1024}" in out
    assert f"fwd_traffic_bytes: {2000 * 1024 * 2 + 500 * 1024}" in out


def test_counters_summary_lists_every_counter(tmp_path, capsys):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    a = _write_csv(tmp_path / "a.csv", hdr, [[STATE, "TCC_HIT_sum", 130e6], [STATE, "TCC_HIT_sum", 132e6],
                                             [STATE, "TCC_MISS_sum", 22e6], [OTHER, "TCC_MISS_sum", 5e6]])
    b = _write_csv(tmp_path / "b.csv", hdr, [[STATE, "TCP_TCC_READ_REQ_sum", 137e6]])
    bench.summarize("counters", [a, b], "t", [])
    out = capsys.readouterr().out
    row = [l for l in out.splitlines() if l.strip().startswith("state_split_kernel")]
    assert len(row) == 1
    assert row[0].split()[-3:] == ["131.000", "22.000", "137.000"]
    assert "elementwise" not in out
