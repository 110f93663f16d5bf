"""The seeded generator: published known answers, value ranges and distributions."""
import math

import numpy as np
import pytest

import synth


def test_splitmix64_known_answer():
    # SplitMix64 seeded with 0 (Vigna's splitmix64.c): its first three outputs
    assert [int(v) for v in synth.stream(0, 3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    # counter-based: any window of the sequence is the same values
    assert np.array_equal(synth.stream(12345, 10, start=5), synth.stream(12345, 15)[5:])


def test_keys_distinct_and_stable():
    ks = {synth.key(7, l, kind, e) for l in range(4) for kind in range(1, 12) for e in range(40)}
    assert len(ks) == 4 * 11 * 40
    assert synth.key(1, 2, 3) == synth.key(1, 2, 3)


def test_record_regions_and_ranges():
    H, I = 256, 128
    rec = synth.expert_record(0xB17E0001, 0, 5, H, I)
    assert rec.size == synth.record_bytes(H, I) == 3 * H * I * 9 // 16
    nb = synth.nibble_region_bytes(H, I)
    cb = synth.segment_code_bytes(4)
    segs = rec.reshape(-1, cb + synth.PAIR_PART_BYTES)
    assert segs.shape[0] * cb == nb
    codes = segs[:, :cb].reshape(-1)
    nib = np.concatenate([codes & 15, codes >> 4])
    counts = np.bincount(nib, minlength=16)
    exp = nib.size / 16
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert chi2 < 50, chi2  # 15 dof
    sb = np.ascontiguousarray(segs[:, cb:]).reshape(-1).view(np.uint16).view(np.float16).astype(np.float64)
    s, b = sb[0::2], sb[1::2]
    assert s.min() >= float(np.float16(1e-3)) and s.max() <= float(np.float16(1e-2))
    assert b.min() >= float(np.float16(-8e-3)) and b.max() <= 0.0
    # biases that land in the fp16 subnormal range: about 6.1e-5 / 8e-3 of them
    frac = np.mean(np.abs(b) < 2.0 ** -14)
    assert 0.003 < frac < 0.013, frac


@pytest.mark.parametrize("bits", [4, 2])
def test_record_segments_hold_the_two_streams_in_order(bits):
    """The code stream fills each segment's code part in order and the pair
    stream its pair part: re-reading the parts in segment order gives the two
    counter streams back (code bytes are the little-endian bytes of the
    stream's words)."""
    H, I, seed, layer, e = 128, 64, 11, 2, 3
    rec = synth.expert_record(seed, layer, e, H, I, bits)
    cb = synth.segment_code_bytes(bits)
    assert cb == 2048 // (4 // bits)
    segs = rec.reshape(-1, cb + 256)
    assert segs.shape[0] == 3 * H * I // 4096
    nb = synth.nibble_region_bytes(H, I, bits)
    words = synth.stream(synth.key(seed, layer, synth.KIND_NIBBLE, e), nb // 8)
    assert np.array_equal(segs[:, :cb].reshape(-1), words.view(np.uint8))
    pairs = np.ascontiguousarray(segs[:, cb:]).reshape(-1).view(np.uint16)
    npairs = synth.sb_pairs(H, I)
    s = 1e-3 + 9e-3 * synth.unit_uniform(synth.stream(synth.key(seed, layer, synth.KIND_SCALE, e), npairs))
    assert np.array_equal(pairs[0::2], synth.to_f16_bits(s))


def test_records_differ_per_expert_and_layer():
    a = synth.expert_record(1, 0, 0, 64, 64)
    assert not np.array_equal(a, synth.expert_record(1, 0, 1, 64, 64))
    assert not np.array_equal(a, synth.expert_record(1, 1, 0, 64, 64))
    assert np.array_equal(a, synth.expert_record(1, 0, 0, 64, 64))


def test_router_ranges():
    q, rs = synth.router(3, 0, 64, 512)
    assert q.dtype == np.int8 and q.min() >= -127 and q.max() <= 127
    assert abs(q.astype(float).mean()) < 1.0
    s = rs.view(np.float16).astype(float) * 73.6 * math.sqrt(512)
    assert s.min() >= 0.49 and s.max() <= 1.51


def test_activations_normal():
    x = synth.activations(9, 0, 0, 4096, n_tokens=4)
    assert x.shape == (4, 4096)
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1.0) < 0.05
    assert not np.array_equal(x, synth.activations(9, 0, 0, 4096, n_tokens=4, attempt=1))


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-3])
    b = synth.to_bf16_bits(v)
    back = synth.bf16_bits_to_f32(b).astype(np.float64)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to the even mantissa (1.0)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2 ** -6
    assert back[3] == -2.5 and abs(back[4] - 1e-3) <= 2 ** -9 * 1e-3


def test_zipf_targets_realised_through_router(orc):
    """The realised activations reproduce the Gumbel-top-k target's top-8 through
    the oracle's router, and the most popular expert is picked most often."""
    E, H, k = 32, 1024, 8
    q, rs = synth.router(11, 0, E, H)
    W = q.astype(np.float64) * rs.view(np.float16).astype(np.float64)[:, None]
    zr = synth.ZipfRealiser(W, 1.1, 11, 0)
    hits = 0
    counts = np.zeros(E)
    n = 200
    for step in range(n):
        x = zr.activations(step)[0]
        xb = synth.bf16_bits_to_f32(synth.to_bf16_bits(x)).astype(np.float64)
        ids, _, _ = orc.route(q, rs, xb, k)
        t = zr.target(step)
        ref = sorted(range(E), key=lambda e: (-t[e], e))[:k]
        hits += sorted(ids.tolist()) == sorted(ref)
        counts[ids] += 1
        assert abs(x.std() - 1.0) < 0.3
    assert hits >= 0.9 * n, hits
    top = int(np.argmin(synth.zipf_rank_of_expert(11, 0, E)))
    assert counts[top] == counts.max()


def test_selection_bias_is_seeded_and_bounded():
    a = synth.selection_bias(7, 0, 300)
    assert a.dtype == np.float32 and a.shape == (300,)
    assert np.all(a >= -0.05) and np.all(a < 0.05)
    assert np.array_equal(a, synth.selection_bias(7, 0, 300))
    assert not np.array_equal(a, synth.selection_bias(7, 1, 300))
    assert abs(float(a.mean())) < 0.01 and float(a.std()) > 0.02


def test_lookahead_hint_is_a_seeded_noisy_preview():
    x = synth.activations(5, 2, 3, 4096, n_tokens=2)
    assert np.array_equal(synth.lookahead_hint(5, 2, 3, x, 1.0), x)
    h = synth.lookahead_hint(5, 2, 3, x, 0.8)
    assert np.array_equal(h, synth.lookahead_hint(5, 2, 3, x, 0.8))
    assert not np.array_equal(h, synth.lookahead_hint(5, 3, 3, x, 0.8))
    for t in range(2):
        c = np.corrcoef(x[t], h[t])[0, 1]
        assert abs(c - 0.8) < 0.02, c
        assert abs(h[t].std() / x[t].std() - 1.0) < 0.05
    z = synth.lookahead_hint(5, 2, 3, x, 0.0)
    assert abs(np.corrcoef(x[0], z[0])[0, 1]) < 0.05


def test_zipf_routing_histogram_matches_the_marginals(orc):
    """GLM-scale decode routing (Zipf(1.1) over 256 experts, layer 0): the
    oracle's selections over the first 2048 seeded steps, counted per
    popularity rank, equal the stored dump (tests/golden/zipf_glm_layer0.json,
    written by tests/golden/make_zipf_histogram.py) and follow the
    Gumbel-top-8 inclusion probabilities: chi^2 per bin near 1 with every
    rank's count within 4.5 standard deviations (binomial per rank)."""
    import json
    import os
    import sys
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    sys.path.insert(0, here)
    import make_zipf_histogram as mz
    with open(os.path.join(here, "zipf_glm_layer0.json")) as f:
        gold = json.load(f)
    counts = np.array(mz.realised_rank_counts(orc, gold["steps"]))
    assert counts.tolist() == gold["counts_by_rank"]
    p = np.array(gold["expected_inclusion_by_rank"])
    assert abs(p.sum() - 8.0) < 1e-4 and np.all(np.diff(p) < 0.002)  # 8 picks (stored to 6 digits); falls with rank
    n = gold["steps"]
    assert counts.sum() == 8 * n
    z2 = (counts - n * p) ** 2 / (n * p * (1 - p))
    chi2_per_bin = float(z2.sum() / p.size)
    print(f"zipf histogram: chi2 per bin {chi2_per_bin:.3f}, max |z| {np.sqrt(z2.max()):.2f}")
    assert 0.75 < chi2_per_bin < 1.35 and float(np.sqrt(z2.max())) < 4.5
