"""CPU checks of bench.py's contract: the algorithmic work it divides by, the
kernel lists it reports, and its refusal of more than one GPU."""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_prefill_algorithmic_bytes_4k_layer():
    # q, k (16 heads x 128) and v, o (32 heads x 128) in bf16, g and beta in
    # fp32 per (token, v-head), plus the fp32 final state of 32 heads
    per_token = (2 * 16 * 128 + 2 * 32 * 128) * 2 + 2 * 32 * 4
    assert bench.prefill_alg_bytes(4096, 16, 32, 128, 128) == 4096 * per_token + 32 * 128 * 128 * 4 == 103_809_024
    # an initial state read adds one more state
    assert bench.prefill_alg_bytes(4096, 16, 32, 128, 128, state_in=True) == 103_809_024 + 32 * 128 * 128 * 4


def test_prefill_algorithmic_flops_per_chunk_head():
    # triangles counted as triangles at C = 64, d = 128: 8.99 MFLOP per chunk-head
    per_chunk_head = bench.prefill_alg_flops(64, 1, 128, 128)
    assert per_chunk_head == pytest.approx(8_992_085.333, rel=1e-9)
    assert bench.prefill_alg_flops(4096, 32, 128, 128) == pytest.approx(64 * 32 * per_chunk_head)
    # the dense state products alone (3 C d_k d_v multiply-adds) are a lower bound
    assert per_chunk_head > 2 * 3 * 64 * 128 * 128


def test_conv_prepare_and_decode_bytes():
    assert bench.conv_prepare_alg_bytes(4096, 8192, 32) == 4096 * 8192 * 2 * 2 + 8192 * 4 * 4 + 2 * 4096 * 32 * 4
    assert bench.conv_prepare_alg_bytes(4096, 8192, 32) == 135_397_376
    # state read + written once, plus the token's q, k, v, o, g, beta
    assert bench.decode_alg_bytes(64, 16, 32, 128, 128) == 270_024_704
    # fused: state read + written, the raw 8192-channel row, the 3-row window
    # read + written, o, g, beta and the 8192 x 4 fp32 taps
    fused = 2 * 64 * 32 * 128 * 128 * 4 + 64 * 8192 * 2 + 2 * 64 * 3 * 8192 * 2 + 64 * 32 * 128 * 2 \
        + 2 * 64 * 32 * 4 + 8192 * 4 * 4
    assert bench.decode_conv_alg_bytes(64, 16, 32, 128, 128, W=4) == fused == 276_447_232


def test_gated_norm_bytes():
    # o and z read, y written (4096 tokens x 32 heads x 128, bf16), plus the fp32 weight
    assert bench.gated_norm_alg_bytes(4096, 32, 128) == 3 * 4096 * 32 * 128 * 2 + 128 * 4 == 100_663_808


def test_gating_bytes():
    # a, b bf16 in, g, beta fp32 out over 4096 tokens x 32 v-heads, plus A_log and dt_bias
    assert bench.gating_alg_bytes(4096, 32) == 2 * 4096 * 32 * 2 + 2 * 4096 * 32 * 4 + 2 * 32 * 4 == 1_573_120


def test_call_kernels_exist_in_their_sources():
    csrc = os.path.join(ROOT, "linear_attention_delta_amd", "csrc")
    for call, kernels in bench.CALL_KERNELS.items():
        text = "".join(open(os.path.join(csrc, f)).read() for f in bench.KERNEL_SOURCES[call])
        for k in kernels:
            assert re.search(r"__global__[^;{]*\b" + k + r"\(", text), (call, k)
        assert re.fullmatch(r"[0-9a-f]{16}", bench.source_digest(call))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True, text=True,
                       env=e, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_varlen_flops_match_dense_on_whole_chunks():
    # whole chunks: the same as the dense count; a partial chunk counts at its length
    assert bench.prefill_alg_flops_varlen([4096], 32, 128, 128) == pytest.approx(
        bench.prefill_alg_flops(4096, 32, 128, 128))
    assert bench.prefill_alg_flops_varlen([64, 128], 2, 128, 128) == pytest.approx(
        bench.prefill_alg_flops(192, 2, 128, 128))
    tail = bench.prefill_alg_flops_varlen([70], 1, 128, 128) - bench.prefill_alg_flops(64, 1, 128, 128)
    # 6 tokens: 2 (6*5/2*128 + 6*7/2*128 + 6^3/6 + 2*6*5/2*128 + 3*6*128*128 + 6*7/2*128)
    assert tail == pytest.approx(2 * (15 * 128 + 21 * 128 + 36 + 30 * 128 + 3 * 6 * 128 * 128 + 21 * 128))
    assert bench.prefill_alg_flops_varlen([0, 0], 4, 64, 64) == 0


def test_percentiles():
    p = bench.percentiles([1.0, 2.0, 3.0, 4.0, 5.0])
    assert p["mean"] == 3.0 and p["p50"] == 3.0 and p["blocks"] == 5
    assert p["p10"] == pytest.approx(1.4) and p["p90"] == pytest.approx(4.6)
