"""The benchmark's host-side pieces, without a GPU: the single-GPU guard, the
algorithmic byte counts, and the lookahead-hint calibration."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single-GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("bits", [4, 2])
def test_algorithmic_bytes_add_up_to_the_record(bits):
    # gate/up and down parts of a record: codes plus one (scale, bias) pair per 64 weights
    for H, I in [(2816, 704), (6144, 2048), (256, 128)]:
        rec = 3 * H * I * bits // 8 + 3 * H * I // 16
        assert bench.gu_bytes(H, I, bits) + bench.down_bytes(H, I, bits) == rec
        assert bench.gu_bytes(H, I, bits) == 2 * bench.down_bytes(H, I, bits)
    wl = synth.WORKLOADS["gemma_a4b_h2816_e128_l30"]
    rec, shared = (3 * 2816 * 704 * bits // 8 + 3 * 2816 * 704 // 16,
                   3 * 2816 * 2112 * bits // 8 + 3 * 2816 * 2112 // 16)
    assert bench.token_layer_bytes(wl, bits) == 128 * 2816 + 2 * 128 + 8 * rec + shared
    if bits == 4:
        assert bench.token_layer_bytes(wl, bits) == 37_160_192  # router + 8 records + shared


def test_lookahead_recall_grows_with_rho_and_calibration_hits_the_target():
    wl = synth.WORKLOADS["offload_h2816_e256_l40_lfu16"]
    L, S = 4, 12
    xs = np.stack([bench.make_inputs(wl, l, S) for l in range(L)], axis=1)  # [S][L][1][H]
    routers = []
    for l in range(L):
        q, rs = synth.router(wl.seed, l, wl.n_experts, wl.hidden)
        routers.append(q.astype(np.float64) * rs.view(np.float16).astype(np.float64)[:, None])
    steps = list(range(S))
    rec = [bench.lookahead_recall(wl, routers, xs, r, steps) for r in (0.2, 0.6, 0.9, 1.0)]
    assert rec[-1] == 1.0  # the input itself predicts exactly
    assert rec[0] < rec[1] < rec[2] < rec[3]
    rho = bench.calibrate_rho(wl, routers, xs, 0.716, steps)
    assert abs(bench.lookahead_recall(wl, routers, xs, rho, steps) - 0.716) < 0.03


@pytest.mark.parametrize("bits", [4, 2])
def test_launch_bytes_cover_the_token_layer(bits):
    """The three launches' bytes add up to the token-layer total, and with the
    router inside the gate/up launch that launch carries the router's bytes
    (the Gemma-scale figure the roofline quotes: 24,893,696 B with 4-bit
    records)."""
    wl = synth.WORKLOADS["gemma_a4b_h2816_e128_l30"]
    sep = bench.launch_bytes(wl, bits, 1, False)
    fused = bench.launch_bytes(wl, bits, 1, True)
    assert sum(sep.values()) == bench.token_layer_bytes(wl, bits)
    assert fused["gate_up"] == sep["gate_up"] + sep["route"] and fused["down_combine"] == sep["down_combine"]
    assert bench.launch_bytes(wl, bits, 3, True)["gate_up"] == 3 * fused["gate_up"]
    if bits == 4:
        assert fused["gate_up"] == 24_893_696 and sep["route"] == 360_704


def test_graph_chunks_divide_the_timed_steps():
    assert bench.chunk_len(20, 32) == 20 and bench.chunk_len(64, 32) == 32
    assert bench.chunk_len(256, 32) == 32 and bench.chunk_len(37, 32) == 1
    assert bench.chunk_len(48, 16) == 16 and bench.chunk_len(1, 32) == 1
    for K in range(1, 100):
        G = bench.chunk_len(K, 32)
        assert K % G == 0 and G <= 32


def test_selected_record_bytes_at_glm_scale():
    # the eight selected records alone, the second byte column of the decode line
    from bit_routed_expert_moe_amd import record_bytes
    wl = synth.WORKLOADS["glm_h6144_e256_l40_zipf"]
    assert wl.top_k * record_bytes(wl.hidden, wl.inter, 4) == 169_869_312
    assert bench.token_layer_bytes(wl, 4) == 192_676_352
