"""Host checks of the benchmark's bookkeeping: the committed rocprofv3 counter
summaries of the LM-head GEMM (profiles/) still describe the current kernel
sources -- the benchmark reports their HBM traffic only while the source hash
matches, so a kernel change without a new counter run fails here -- and the
calibrated traffic is close to the launch's algorithmic bytes."""
import pytest

bench = pytest.importorskip("bench")


@pytest.mark.parametrize("fp8", [False, True])
def test_recorded_lm_head_traffic_matches_sources(fp8):
    V, H, M = 151936, 5120, 7                      # the B = 1, k = 7 LM head
    if fp8:   # E4M3 codes + fp32 row scales + bf16 hidden states + fp32 logits
        alg = V * H + V * 4 + M * H * 2 + M * V * 4
    else:     # bf16 weights + bf16 hidden states + fp32 logits
        alg = V * H * 2 + M * H * 2 + M * V * 4
    t = bench.recorded_traffic("qwen27b_b1", "fp8" if fp8 else "native")
    assert t is not None, "LM-head counter summary missing or older than the GEMM sources"
    assert 0.98 * alg <= t <= 1.05 * alg, (t, alg)


@pytest.mark.parametrize("weights", ["native", "packed"])
@pytest.mark.parametrize("name,M,H", [("adaptive_b16", 128, 5120), ("b16", 112, 5120),
                                      ("flashnext_b4", 32, 2560)])
def test_recorded_traffic_of_the_batched_workloads(name, M, H, weights):
    """The row-split LM head of the batched workloads, row-major and packed
    weights: counter summary present for the current sources, traffic within
    5 % of the algorithmic bytes."""
    V = 151936
    alg = V * H * 2 + M * H * 2 + M * V * 4
    t = bench.recorded_traffic(name, weights)
    assert t is not None, "LM-head counter summary missing or older than the GEMM sources"
    assert 0.98 * alg <= t <= 1.05 * alg, (t, alg)


@pytest.mark.parametrize("weights", ["native", "packed"])
def test_recorded_traffic_of_the_fused_launch(weights):
    """The fc and the LM head in one launch (flashnext_b4): summary present for
    the current sources, traffic within 5 % of the algorithmic bytes."""
    V, H, M, rows, T = 151936, 2560, 32, 36, 5
    alg = V * H * 2 + M * H * 2 + M * V * 4 + (H * T * H + rows * T * H + rows * H) * 2
    t = bench.recorded_traffic("flashnext_b4", weights, "fc_lm_head_gemm")
    assert t is not None, "fused-launch counter summary missing or older than the GEMM sources"
    assert 0.98 * alg <= t <= 1.05 * alg, (t, alg)
