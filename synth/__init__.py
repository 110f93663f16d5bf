"""Seeded synthetic inputs for the routed-expert MoE layer.

This package is shared by the GPU path's tests/bench and by the oracle's tests.
It holds random draws and byte filling only: nothing in it computes a router
logit, a top-k, a dequantised weight or an FFN output.  Everything is derived
from one counter-based generator, SplitMix64 (Steele, Lea and Flood,
"Fast Splittable Pseudorandom Number Generators", OOPSLA 2014; the output
function is the public-domain ``splitmix64.c`` finaliser by S. Vigna):

    state_i  = key + (i + 1) * 0x9E3779B97F4A7C15          (mod 2^64)
    out_i    = mix64(state_i)
    mix64(z) = z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
               z ^= z >> 27; z *= 0x94D049BB133111EB; z ^ (z >> 31)

``synth/fill.hip`` implements the same definition on the GPU for the large
expert pools; ``tests/test_synth.py`` checks the two agree byte for byte.

Stream keys: ``key(seed, layer, kind, index[, attempt])`` folds each part p as
``k = mix64((k ^ p) + GAMMA)`` starting from k = 0.

Value recipes (every float goes double -> float32 -> target type, each step
round-to-nearest-even; the double arithmetic is one multiply then one add, no
fused multiply-add):
  code bytes       little-endian bytes of out_i: byte p = byte (p & 7) of out_{p >> 3}
  scale s          fp16(fp32(1e-3 + 9e-3 * U))          U = (out >> 11) * 2^-53
  bias  b          fp16(fp32(-8e-3 * U))
  router int8      ((out >> 32) mod 255) - 127
  router scale     fp16(fp32((0.5 + U) / (73.6 * sqrt(H))))
  activations      Box-Muller: sqrt(-2 ln U1) cos(2 pi U2), U1 = ((out1 >> 11) + 0.5) 2^-53
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB

# stream kinds
KIND_NIBBLE = 1
KIND_SCALE = 2
KIND_BIAS = 3
KIND_ROUTER_Q = 4
KIND_ROUTER_S = 5
KIND_X1 = 6
KIND_X2 = 7
KIND_PERM = 8
KIND_GUMBEL = 9
KIND_Z1 = 10
KIND_Z2 = 11
KIND_SEL_BIAS = 12
KIND_HINT1 = 13
KIND_HINT2 = 14
SHARED_INDEX = 0xFFFF  # expert index used for the shared expert's streams


def mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * _M1) & MASK64
    z = ((z ^ (z >> 27)) * _M2) & MASK64
    return z ^ (z >> 31)


def mix64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    z ^= z >> np.uint64(30)
    z *= np.uint64(_M1)
    z ^= z >> np.uint64(27)
    z *= np.uint64(_M2)
    z ^= z >> np.uint64(31)
    return z


def key(*parts: int) -> int:
    k = 0
    for p in parts:
        k = mix64_int(((k ^ (int(p) & MASK64)) + GAMMA) & MASK64)
    return k


def stream(k: int, n: int, start: int = 0) -> np.ndarray:
    """out_i for i in [start, start + n) of the SplitMix64 sequence keyed by k."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + 1 + n, dtype=np.uint64)
        z = np.uint64(k) + idx * np.uint64(GAMMA)
    return mix64(z)


def unit_uniform(u: np.ndarray) -> np.ndarray:
    """U in [0, 1) with 53 random bits."""
    return (u >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def to_f16_bits(v: np.ndarray) -> np.ndarray:
    return v.astype(np.float32).astype(np.float16).view(np.uint16)


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """double -> fp32 (RNE) -> bf16 (RNE); inputs are finite."""
    b = np.ascontiguousarray(v.astype(np.float32)).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# expert records: a sequence of equal segments, each SEGMENT_CODE_BYTES of
# weight codes followed by 256 bytes (64 pairs) of (scale, bias) fp16 pairs.
# The code stream fills the code parts in order and the pair stream the pair
# parts; which weights a code or a pair belongs to is the layout's business,
# not the generator's.
# ---------------------------------------------------------------------------
PAIR_PART_BYTES = 256


def segment_code_bytes(bits: int = 4) -> int:
    """Code bytes per segment: 64 rows x 64 inputs of `bits`-wide codes."""
    return 64 * 64 * bits // 8


def nibble_region_bytes(hidden: int, inter: int, bits: int = 4) -> int:
    """Code bytes of a record (4-bit nibbles, or 2-bit codes), all segments."""
    return 3 * hidden * inter * bits // 8


def sb_pairs(hidden: int, inter: int) -> int:
    return 3 * hidden * inter // 64


def record_bytes(hidden: int, inter: int, bits: int = 4) -> int:
    return nibble_region_bytes(hidden, inter, bits) + 4 * sb_pairs(hidden, inter)


def expert_record(seed: int, layer: int, expert: int, hidden: int, inter: int,
                  bits: int = 4) -> np.ndarray:
    """One packed expert record (uint8), generated on the CPU."""
    nb = nibble_region_bytes(hidden, inter, bits)
    npairs = sb_pairs(hidden, inter)
    codes = stream(key(seed, layer, KIND_NIBBLE, expert), nb // 8).view(np.uint8)
    s = 1e-3 + 9e-3 * unit_uniform(stream(key(seed, layer, KIND_SCALE, expert), npairs))
    b = -8e-3 * unit_uniform(stream(key(seed, layer, KIND_BIAS, expert), npairs))
    sb = np.empty(2 * npairs, dtype=np.uint16)
    sb[0::2] = to_f16_bits(s)
    sb[1::2] = to_f16_bits(b)
    cb = segment_code_bytes(bits)
    nseg = nb // cb
    assert nseg * PAIR_PART_BYTES == 4 * npairs
    out = np.empty((nseg, cb + PAIR_PART_BYTES), dtype=np.uint8)
    out[:, :cb] = codes.reshape(nseg, cb)
    out[:, cb:] = sb.view(np.uint8).reshape(nseg, PAIR_PART_BYTES)
    return out.reshape(-1)


def router(seed: int, layer: int, n_experts: int, hidden: int):
    """int8 router rows [E][H] and their fp16 scales [E] (as uint16 bits)."""
    u = stream(key(seed, layer, KIND_ROUTER_Q, 0), n_experts * hidden)
    q = ((u >> np.uint64(32)) % np.uint64(255)).astype(np.int32) - 127
    rs = (0.5 + unit_uniform(stream(key(seed, layer, KIND_ROUTER_S, 0), n_experts))) / (
        73.6 * math.sqrt(hidden))
    return q.astype(np.int8).reshape(n_experts, hidden), to_f16_bits(rs)


def selection_bias(seed: int, layer: int, n_experts: int, half_width: float = 0.05) -> np.ndarray:
    """Per-expert selection bias of the sigmoid router, float32 uniform on
    [-half_width, half_width) (the pages give no values; any fixed seeded draw
    exercises the path)."""
    u = unit_uniform(stream(key(seed, layer, KIND_SEL_BIAS, 0), n_experts))
    return ((2.0 * u - 1.0) * half_width).astype(np.float32)


def normal(k1: int, k2: int, n: int) -> np.ndarray:
    u1 = ((stream(k1, n) >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)
    u2 = unit_uniform(stream(k2, n))
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def activations(seed: int, layer: int, step: int, hidden: int, n_tokens: int = 1,
                attempt: int = 0) -> np.ndarray:
    """N(0,1) activations for one (layer, step) as float64 [n_tokens][hidden]."""
    n = n_tokens * hidden
    x = normal(key(seed, layer, KIND_X1, step, attempt), key(seed, layer, KIND_X2, step, attempt), n)
    return x.reshape(n_tokens, hidden)


def lookahead_hint(seed: int, layer: int, step: int, x: np.ndarray, rho: float) -> np.ndarray:
    """A noisy preview of the activations x ([n][H] float64) as a lookahead
    router sees them a layer early: rho * x + sqrt(1 - rho^2) * std(x) * z per
    token, z ~ N(0, 1) seeded per (layer, step).  In a residual stream the next
    layer's input is the current state plus the current layer's update; rho
    sets how far that update moves it.  The pages give the recall such a
    preview reaches on a real model, not rho, so callers pick rho for a recall."""
    x = np.asarray(x, dtype=np.float64)
    z = normal(key(seed, layer, KIND_HINT1, step), key(seed, layer, KIND_HINT2, step), x.size)
    z = z.reshape(x.shape)
    sd = x.std(axis=-1, keepdims=True)
    return rho * x + math.sqrt(max(0.0, 1.0 - rho * rho)) * sd * z


def quantize_act(x: np.ndarray, act: str) -> np.ndarray:
    """Round float64 activations to the activation dtype; returns the raw array
    (float32 for 'f32', uint16 bf16 bits for 'bf16')."""
    if act == "f32":
        return x.astype(np.float32)
    if act == "bf16":
        return to_bf16_bits(x)
    raise ValueError(act)


# ---------------------------------------------------------------------------
# Zipf(s) routing realised through the router (input shaping only): a seeded
# popularity permutation per layer, Gumbel-perturbed log-popularities as target
# logits, and an activation vector whose router response equals the target in
# the least-squares sense.  The router's response is recomputed independently
# by whoever consumes these inputs.
# ---------------------------------------------------------------------------

def zipf_rank_of_expert(seed: int, layer: int, n_experts: int) -> np.ndarray:
    """rank[e] in 1..E: popularity rank of expert e in this layer."""
    order = np.argsort(stream(key(seed, layer, KIND_PERM, 0), n_experts), kind="stable")
    rank = np.empty(n_experts, dtype=np.int64)
    rank[order] = np.arange(1, n_experts + 1)
    return rank


def zipf_probs(n_experts: int, s: float) -> np.ndarray:
    p = np.arange(1, n_experts + 1, dtype=np.float64) ** (-s)
    return p / p.sum()


def gumbel(k: int, n: int) -> np.ndarray:
    u = ((stream(k, n) >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)
    return -np.log(-np.log(u))


class ZipfRealiser:
    """Builds activations whose router logits follow Zipf(s)-popular Gumbel-top-k
    targets.  ``router_dense`` is the caller's dense [E][H] router (the int8 rows
    times their scales) - used here only to aim the draw."""

    def __init__(self, router_dense: np.ndarray, s: float, seed: int, layer: int):
        self.E, self.H = router_dense.shape
        self.W = router_dense
        q, r = np.linalg.qr(router_dense.T)  # W^T = Q R
        self.Q, self.R = q, r
        self.logp = np.log(zipf_probs(self.E, s))[zipf_rank_of_expert(seed, layer, self.E) - 1]
        self.seed, self.layer = seed, layer

    def target(self, step: int, attempt: int = 0) -> np.ndarray:
        g = gumbel(key(self.seed, self.layer, KIND_GUMBEL, step, attempt), self.E)
        t = self.logp + g
        return t - t.mean()

    def activations(self, step: int, attempt: int = 0) -> np.ndarray:
        import scipy.linalg as sla
        t = self.target(step, attempt)
        z = normal(key(self.seed, self.layer, KIND_Z1, step, attempt),
                   key(self.seed, self.layer, KIND_Z2, step, attempt), self.H)
        resid = t - self.W @ z
        # minimum-norm d with W d = resid:  W = R^T Q^T  ->  d = Q R^{-T} resid
        d = self.Q @ sla.solve_triangular(self.R.T, resid, lower=True)
        return (z + d)[None, :]

    def activations_batch(self, steps, attempt: int = 0) -> np.ndarray:
        """activations(step, attempt)[0] for every step, as one [S][H] array
        (the same draws; the least-squares step runs on all of them at once, so
        values may differ from the one-step form in the last bits)."""
        import scipy.linalg as sla
        steps = list(steps)
        t = np.stack([self.target(s, attempt) for s in steps])
        z = np.stack([normal(key(self.seed, self.layer, KIND_Z1, s, attempt),
                             key(self.seed, self.layer, KIND_Z2, s, attempt), self.H) for s in steps])
        resid = t - z @ self.W.T
        d = sla.solve_triangular(self.R.T, resid.T, lower=True)
        return z + (self.Q @ d).T


# ---------------------------------------------------------------------------
# workloads (shapes and recipes of the pages' configurations)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    hidden: int
    n_experts: int
    inter: int
    top_k: int
    shared_inter: int
    act: str            # "f32" or "bf16"
    n_layers: int
    n_tokens: int       # tokens per step (1 = decode, 128 = prefill chunk)
    steps: int
    routing: str        # "natural" (x ~ N(0,1) through the router), "zipf" or
                        # "uniform" (Gumbel-top-k targets realised through the
                        # router; uniform = Zipf with s = 0)
    zipf_s: float = 0.0
    n_slots: int = 0    # HBM expert slots per layer (0 = fully resident)
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def record_bytes(self) -> int:
        return record_bytes(self.hidden, self.inter)

    @property
    def shared_record_bytes(self) -> int:
        return record_bytes(self.hidden, self.shared_inter) if self.shared_inter else 0

    @property
    def router_bytes(self) -> int:
        return self.n_experts * self.hidden + 2 * self.n_experts

    @property
    def token_layer_bytes(self) -> int:
        """Algorithmic HBM bytes of one decode token through one layer: the
        router, the top_k selected records and the shared record."""
        return self.router_bytes + self.top_k * self.record_bytes + self.shared_record_bytes


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_h256_e32", 256, 32, 128, 8, 256, "f32", 1, 1, 1, "natural",
                 seed=0xB17E0001, note="tiny single layer, fp32 activations, 1 token"),
        Workload("gemma_a4b_h2816_e128_l30", 2816, 128, 704, 8, 2112, "bf16", 30, 1, 256,
                 "natural", seed=0xB17E0002,
                 note="Gemma-4-A4B-scale 30-layer decode stack, 256 decode steps"),
        Workload("glm_h6144_e256_l40_zipf", 6144, 256, 2048, 8, 2048, "bf16", 40, 1, 256,
                 "zipf", zipf_s=1.1, seed=0xB17E0003,
                 note="GLM-scale 40-layer decode, Zipf(1.1) routing"),
        Workload("glm_prefill_h6144_e256_t128", 6144, 256, 2048, 8, 2048, "bf16", 1, 128, 1,
                 "uniform", zipf_s=0.0, seed=0xB17E0004,
                 note="GLM-scale 128-token prefill chunk, uniform random routing"),
        Workload("offload_h2816_e256_l40_lfu16", 2816, 256, 704, 8, 2112, "bf16", 40, 1, 512,
                 "zipf", zipf_s=1.1, n_slots=16, seed=0xB17E0005,
                 note="out-of-core decode: 16-slot LFU per layer, pinned host pool"),
    ]
}
