"""Writes tests/golden/zipf_glm_layer0.json: how often each popularity rank of
the GLM-scale decode workload (hidden 6144, 256 experts, Zipf(1.1), layer 0)
is selected over its first STEPS decode steps, and the inclusion probability
each rank should have.

* Realised counts: the seeded activations of synth.ZipfRealiser (as bench.py
  feeds them), quantised to bf16, routed by the oracle (exact top-8 of its
  float64 logits).  Inputs come from synth/, selections from oracle/ only.
* Expected: the probability that a rank is among 8 draws without replacement
  proportional to rank^-1.1 (Gumbel-top-8 of the log-popularities), by a Monte
  Carlo of MC_DRAWS draws on numpy's own generator (independent of synth's
  counter streams).

Run: python tests/golden/make_zipf_histogram.py
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

STEPS = 2048
MC_DRAWS = 400_000
OUT = os.path.join(HERE, "zipf_glm_layer0.json")


def realised_rank_counts(orc, steps: int = STEPS) -> list[int]:
    import synth
    wl = synth.WORKLOADS["glm_h6144_e256_l40_zipf"]
    rq, rs = synth.router(wl.seed, 0, wl.n_experts, wl.hidden)
    W = rq.astype(np.float64) * rs.view(np.float16).astype(np.float64)[:, None]
    zr = synth.ZipfRealiser(W, wl.zipf_s, wl.seed, 0)
    xs = synth.quantize_act(zr.activations_batch(range(steps)), wl.act)
    rank = synth.zipf_rank_of_expert(wl.seed, 0, wl.n_experts)
    counts = np.zeros(wl.n_experts, dtype=np.int64)
    for t in range(steps):
        ids, _, _ = orc.route(rq, rs, orc.act_to_f64(wl.act, xs[t]), wl.top_k)
        np.add.at(counts, rank[ids] - 1, 1)
    return counts.tolist()


def expected_inclusion(n_experts: int = 256, s: float = 1.1, k: int = 8, draws: int = MC_DRAWS,
                       seed: int = 20261202) -> list[float]:
    rng = np.random.default_rng(seed)
    logp = -s * np.log(np.arange(1, n_experts + 1, dtype=np.float64))
    hits = np.zeros(n_experts, dtype=np.int64)
    for c0 in range(0, draws, 20_000):
        g = rng.gumbel(size=(min(20_000, draws - c0), n_experts)) + logp
        top = np.argpartition(-g, k, axis=1)[:, :k]
        np.add.at(hits, top.reshape(-1), 1)
    return (hits / draws).tolist()


def main():
    import oracle
    orc = oracle.default()
    data = {
        "_about": "Selections per popularity rank (1 = most popular) of the GLM-scale decode workload's "
                  "layer 0 over its first steps, routed by the oracle, and the Gumbel-top-8 inclusion "
                  "probability of each rank (Monte Carlo, numpy's generator). Written by "
                  "tests/golden/make_zipf_histogram.py.",
        "steps": STEPS, "top_k": 8, "zipf_s": 1.1, "mc_draws": MC_DRAWS,
        "counts_by_rank": realised_rank_counts(orc),
        "expected_inclusion_by_rank": [round(p, 6) for p in expected_inclusion()],
    }
    with open(OUT, "w") as f:
        json.dump(data, f, indent=1)
    print(OUT)


if __name__ == "__main__":
    main()
