"""Pins of the CPU oracle against things other than itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch.  They are run against the real oracle (tests/test_oracle_pins.py)
and against deliberately broken copies of it (tests/test_oracle_mutants.py),
which must each fail at least one pin.

What they pin to:
  * numpy's own IEEE half conversion and bit-level bf16 widening
  * an independently written packer and the dense matrices it packs
  * closed forms (constant weights, zero scales, one-hot inputs)
  * a dense SwiGLU computed with library matmuls and scipy's logistic
  * exact integer arithmetic for the router
  * brute-force sorting for top-k, scipy's softmax for the gates
  * a hand-worked gate example (softmax and sigmoid routers)
  * sizes printed on the pages (tests/golden/page_sizes.json)
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.special import expit, softmax

from _packer import DenseExpert, pack_record

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, rtol=1e-12, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= rtol * scale + atol, f"{what}: max abs err {err:.3e} vs scale {scale:.3e}"


def pin_f16_decode(orc):
    """Every finite binary16 pattern decodes like numpy's float16 -> float64."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin]), "fp16 decode differs from numpy"
    assert np.all(np.isinf(got[np.isinf(ref)])) and np.all(np.isnan(got[np.isnan(ref)]))
    assert orc.f16(0x0001) == 2.0 ** -24 and orc.f16(0x7BFF) == 65504.0 and orc.f16(0xC000) == -2.0


def pin_bf16_decode(orc):
    """bf16 is the upper half of binary32 (checked on a spread of patterns)."""
    rng = np.random.default_rng(1)
    bits = np.concatenate([rng.integers(0, 65536, 4000), [0, 0x3F80, 0xBF80, 0x0001, 0x7F7F]])
    for b in bits:
        ref = float(np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0])
        got = orc.bf16(int(b))
        assert got == ref or (math.isnan(got) and math.isnan(ref)), hex(int(b))
    x = np.array([0x3F80, 0xC040], dtype=np.uint16)
    assert np.array_equal(orc.act_to_f64("bf16", x), [1.0, -3.0])


def pin_dequant_matches_packer(orc):
    """Dense dequantisation of packed bytes equals scale*q+bias of the source."""
    rng = np.random.default_rng(2)
    for H, I in [(64, 64), (128, 192), (192, 128), (256, 128)]:
        ex = DenseExpert(H, I, rng, s_range=(-0.02, 0.02), b_range=(-0.01, 0.01))
        assert orc.record_bytes(H, I) == ex.rec.size == 3 * H * I * 9 // 16
        G, U, D = orc.dequant_record(H, I, ex.rec)
        assert np.array_equal(G, ex.G) and np.array_equal(U, ex.U) and np.array_equal(D, ex.D), \
            f"dequant mismatch at H={H} I={I}"


def pin_two_bit_format(orc):
    """The 2-bit variant: dequantisation of packed bytes equals scale*q+bias of
    the source (q in 0..3), the record is 15HI/16 bytes, one expert equals the
    dense SwiGLU with library matmuls, and constant codes give the closed form."""
    rng = np.random.default_rng(22)
    for H, I in [(64, 64), (128, 192), (256, 128), (320, 64)]:
        ex = DenseExpert(H, I, rng, s_range=(-0.02, 0.02), b_range=(-0.01, 0.01), bits=2)
        assert orc.record_bytes(H, I, bits=2) == ex.rec.size == 15 * H * I // 16
        G, U, D = orc.dequant_record(H, I, ex.rec, bits=2)
        assert np.array_equal(G, ex.G) and np.array_equal(U, ex.U) and np.array_equal(D, ex.D), \
            f"2-bit dequant mismatch at H={H} I={I}"
        x = rng.standard_normal(H)
        _close(orc.expert_ffn(H, I, ex.rec, x, bits=2), ex.ffn(x), 1e-12, what=f"2-bit ffn H={H}")
    H, I, c, s, b = 128, 64, 3, 2.0 ** -6, -(2.0 ** -9)
    f16 = lambda v, shape: np.full(shape, np.float16(v)).view(np.uint16)
    sb = (f16(s, (I, H // 64)), f16(b, (I, H // 64)), f16(s, (I, H // 64)), f16(b, (I, H // 64)),
          f16(s, (H, I // 64)), f16(b, (H, I // 64)))
    ex = DenseExpert(H, I, rng, qG=np.full((I, H), c), qU=np.full((I, H), c),
                     qD=np.full((H, I), c), sb=sb, bits=2)
    x = rng.standard_normal(H)
    gamma = (s * c + b) * x.sum()
    h = gamma / (1.0 + math.exp(-gamma)) * gamma
    _close(orc.expert_ffn(H, I, ex.rec, x, bits=2), np.full(H, (s * c + b) * I * h), 1e-12,
           what="2-bit closed form")


def pin_one_hot_columns(orc):
    """x = e_k reads out column k of G and U exactly; y reads D times h."""
    rng = np.random.default_rng(3)
    H, I = 128, 128
    ex = DenseExpert(H, I, rng)
    for k in [0, 1, 31, 32, 63, 64, 95, 127]:
        x = np.zeros(H); x[k] = 1.0
        y, g, u, h = orc.expert_ffn(H, I, ex.rec, x, intermediates=True)
        assert np.array_equal(g, ex.G[:, k]) and np.array_equal(u, ex.U[:, k]), f"column {k}"
        _close(h, g * expit(g) * u, 1e-15, what="h")
        _close(y, ex.D @ h, 1e-13, what="y")


def pin_constant_closed_form(orc):
    """q, scale, bias constant per matrix:  g = u = (s c + b) sum(x) =: gamma,
    h = silu(gamma) gamma, y_o = (s' c' + b') * I * h."""
    rng = np.random.default_rng(4)
    H, I = 192, 128
    c, s, b = 5, 2.0 ** -7, -(2.0 ** -9)
    c2, s2, b2 = 9, 2.0 ** -8, 2.0 ** -10
    f16 = lambda v, shape: np.full(shape, np.float16(v)).view(np.uint16)
    sb = (f16(s, (I, H // 64)), f16(b, (I, H // 64)), f16(s, (I, H // 64)), f16(b, (I, H // 64)),
          f16(s2, (H, I // 64)), f16(b2, (H, I // 64)))
    ex = DenseExpert(H, I, rng, qG=np.full((I, H), c), qU=np.full((I, H), c),
                     qD=np.full((H, I), c2), sb=sb)
    x = rng.standard_normal(H)
    gamma = (s * c + b) * x.sum()
    h = gamma / (1.0 + math.exp(-gamma)) * gamma
    y_ref = np.full(H, (s2 * c2 + b2) * I * h)
    y, g, u, hh = orc.expert_ffn(H, I, ex.rec, x, intermediates=True)
    _close(g, np.full(I, gamma), 1e-12, what="g")
    _close(u, np.full(I, gamma), 1e-12, what="u")
    _close(y, y_ref, 1e-12, what="y")


def pin_zero_scale(orc):
    """scale = 0: each row reduces to sum over groups of bias_g * (sum of x in g)."""
    rng = np.random.default_rng(5)
    H, I = 256, 64
    zero = lambda shape: np.zeros(shape, dtype=np.uint16)
    bias = lambda shape: rng.uniform(-0.05, 0.05, shape).astype(np.float16).view(np.uint16)
    bG, bU, bD = bias((I, H // 64)), bias((I, H // 64)), bias((H, I // 64))
    ex = DenseExpert(H, I, rng, sb=(zero((I, H // 64)), bG, zero((I, H // 64)), bU,
                                    zero((H, I // 64)), bD))
    x = rng.standard_normal(H)
    xs = x.reshape(H // 64, 64).sum(axis=1)
    g_ref = bG.view(np.float16).astype(np.float64) @ xs
    u_ref = bU.view(np.float16).astype(np.float64) @ xs
    h_ref = g_ref * expit(g_ref) * u_ref
    y_ref = bD.view(np.float16).astype(np.float64) @ h_ref.reshape(I // 64, 64).sum(axis=1)
    y, g, u, h = orc.expert_ffn(H, I, ex.rec, x, intermediates=True)
    _close(g, g_ref, 1e-12, what="g"); _close(u, u_ref, 1e-12, what="u")
    _close(y, y_ref, 1e-12, what="y")


def pin_dense_swiglu(orc):
    """One expert equals the dense SwiGLU  D (silu(G x) * (U x))  computed with
    library matmuls on the dense matrices (the k = 1, weight 1, no-shared case)."""
    rng = np.random.default_rng(6)
    for H, I in [(64, 64), (256, 128), (320, 192)]:
        ex = DenseExpert(H, I, rng)
        x = rng.standard_normal(H)
        _close(orc.expert_ffn(H, I, ex.rec, x), ex.ffn(x), 1e-12, what=f"ffn H={H} I={I}")
        # the same through the whole-layer entry with k = 1 and no shared expert
        E = 3
        others = [DenseExpert(H, I, rng) for _ in range(E - 1)]
        pool = np.concatenate([others[0].rec, ex.rec, others[1].rec])
        rq = np.zeros((E, H), dtype=np.int8); rq[1, :] = 1
        rs = np.full(E, np.float16(1.0)).view(np.uint16)
        xp = np.abs(x)
        ids, w, y, _ = orc.layer_token(rq, rs, pool, None, I, 0, 1, xp)
        assert ids.tolist() == [1] and w.tolist() == [1.0]
        _close(y, ex.ffn(xp), 1e-12, what="layer k=1")


def pin_router_integer(orc):
    """Integer activations make the row sums exact integers; the logit is the
    fp16 scale times that integer, exactly representable in double."""
    rng = np.random.default_rng(7)
    E, H = 16, 512
    rq = rng.integers(-127, 128, (E, H)).astype(np.int8)
    rs = rng.uniform(0.5, 1.5, E).astype(np.float16).view(np.uint16)
    x = rng.integers(-8, 9, H)
    got = orc.router_logits(rq, rs, x.astype(np.float64))
    for e in range(E):
        exact = sum(int(a) * int(b) for a, b in zip(rq[e], x))
        assert got[e] == float(np.uint16(rs[e]).view(np.float16)) * exact, f"row {e}"


def pin_topk_bruteforce(orc):
    """Top-k equals the first k of a brute-force sort by (-logit, id), ties included."""
    rng = np.random.default_rng(8)
    for trial in range(200):
        E = int(rng.integers(1, 300))
        k = int(rng.integers(1, E + 1))
        lg = np.round(rng.standard_normal(E), 1)  # many exact ties
        ref = sorted(range(E), key=lambda e: (-lg[e], e))[:k]
        assert orc.select_topk(lg, k).tolist() == ref, f"trial {trial}"
    assert orc.select_topk(np.array([1.0, 3.0, 3.0, 2.0]), 2).tolist() == [1, 2]


def pin_gates(orc):
    """Hand-worked example: logits (0, ln 2, ln 3), k = 2 -> ids (2, 1), w = (3/5, 2/5).
    k = E reduces to scipy's softmax; k = 1 gives weight 1; shift invariance."""
    lg = np.array([0.0, math.log(2.0), math.log(3.0)])
    ids = orc.select_topk(lg, 2)
    w = orc.softmax_gates(lg[ids])
    assert ids.tolist() == [2, 1]
    _close(w, [0.6, 0.4], 0, 1e-15, what="worked example")
    rng = np.random.default_rng(9)
    for E in [1, 4, 32, 257]:
        lg = rng.standard_normal(E) * 3
        ids = orc.select_topk(lg, E)
        _close(orc.softmax_gates(lg[ids]), softmax(lg[ids]), 1e-14, what="k=E softmax")
        _close(orc.softmax_gates(lg[ids] + 123.25), softmax(lg[ids]), 1e-13, what="shift")
    assert orc.softmax_gates(np.array([-4.2])).tolist() == [1.0]


def pin_sigmoid_router(orc):
    """Sigmoid router.  Hand-worked: logits (ln 3, -ln 3, 5, 6) with bias
    (10, 10, 0, 0), k = 2, scale 2.5 -> ids (0, 1) (the bias decides the
    selection) and gates from the unbiased scores 3/4 and 1/4: 2.5 * (3/4, 1/4).
    Zero bias selects as the softmax router (the logistic is increasing);
    equal logits give scale / k each with the lowest ids; k = 1 gives scale;
    with random bias the selection is a brute-force sort by (-(logistic + bias),
    id) and the gates sum to the scale."""
    lg = np.array([math.log(3.0), -math.log(3.0), 5.0, 6.0])
    ids, w = orc.sigmoid_route(lg, 2, np.array([10.0, 10.0, 0.0, 0.0]), 2.5)
    assert ids.tolist() == [0, 1]
    _close(w, [1.875, 0.625], 0, 1e-15, what="worked example")
    rng = np.random.default_rng(21)
    for trial in range(100):
        E = int(rng.integers(1, 300)); k = int(rng.integers(1, min(E, 16) + 1))
        lg = rng.standard_normal(E) * 2
        ids, w = orc.sigmoid_route(lg, k, None, 1.0)
        assert ids.tolist() == orc.select_topk(lg, k).tolist(), f"zero bias, trial {trial}"
        b = np.round(rng.standard_normal(E) * 0.3, 1)
        key = expit(lg) + b
        ids, w = orc.sigmoid_route(lg, k, b, 1.7)
        assert ids.tolist() == sorted(range(E), key=lambda e: (-key[e], e))[:k], f"bias, trial {trial}"
        _close(np.sum(w), 1.7, 1e-14, what="gates sum to the scale")
        _close(w / w[0], expit(lg[ids]) / expit(lg[ids[0]]), 1e-13, what="gates from unbiased scores")
    ids, w = orc.sigmoid_route(np.full(10, 0.3), 4, None, 3.0)
    assert ids.tolist() == [0, 1, 2, 3]
    _close(w, np.full(4, 0.75), 0, 1e-15, what="equal logits")
    assert orc.sigmoid_route(np.array([-7.0, 2.0]), 1, None, 2.5)[1].tolist() == [2.5]


def pin_silu(orc):
    """silu(0) = 0; silu(v) - silu(-v) = v; silu(v) = v * logistic(v)."""
    assert orc.silu(0.0) == 0.0
    for v in [-30.0, -2.5, -1e-3, 0.7, 3.0, 25.0]:
        _close(orc.silu(v) - orc.silu(-v), v, 1e-15, what="odd part")
        _close(orc.silu(v), v * expit(v), 1e-15, what="logistic")


def pin_combine(orc):
    """Combine is w^T Y + y_shared: checked against a matmul, under permutation
    of the (expert, weight) pairs, and for linearity in w."""
    rng = np.random.default_rng(10)
    k, H = 8, 96
    Y = rng.standard_normal((k, H)); ys = rng.standard_normal(H); w = rng.dirichlet(np.ones(k))
    _close(orc.combine(w, Y, ys), w @ Y + ys, 1e-14, what="matmul")
    _close(orc.combine(w, Y, None), w @ Y, 1e-14, what="no shared")
    p = rng.permutation(k)
    _close(orc.combine(w[p], Y[p], ys), orc.combine(w, Y, ys), 1e-14, what="permutation")
    w2 = rng.dirichlet(np.ones(k))
    _close(orc.combine(w + w2, Y, None), orc.combine(w, Y, None) + orc.combine(w2, Y, None),
           1e-14, what="linearity")
    _close(orc.combine(np.zeros(k), Y, ys), ys, 0, 0, what="shared only")


def pin_layer_token_dense(orc):
    """A whole layer on a packed pool equals its dense composition: router by
    matmul of int8 rows times scales, brute-force top-k, scipy softmax gates,
    dense SwiGLU per expert, weighted sum plus the shared expert."""
    rng = np.random.default_rng(11)
    H, I, Is, E, k = 128, 64, 128, 12, 4
    experts = [DenseExpert(H, I, rng) for _ in range(E)]
    shared = DenseExpert(H, Is, rng)
    pool = np.concatenate([e.rec for e in experts])
    rq = rng.integers(-127, 128, (E, H)).astype(np.int8)
    rs = (rng.uniform(0.5, 1.5, E) / (73.6 * math.sqrt(H))).astype(np.float16).view(np.uint16)
    for _ in range(5):
        x = rng.standard_normal(H)
        lg = (rq.astype(np.float64) @ x) * rs.view(np.float16).astype(np.float64)
        ref_ids = sorted(range(E), key=lambda e: (-lg[e], e))[:k]
        ref_w = softmax(lg[ref_ids])
        ref_y = sum(wj * experts[e].ffn(x) for wj, e in zip(ref_w, ref_ids)) + shared.ffn(x)
        ids, w, y, lg2 = orc.layer_token(rq, rs, pool, shared.rec, I, Is, k, x)
        assert ids.tolist() == ref_ids
        _close(lg2, lg, 1e-13, what="logits")
        _close(w, ref_w, 1e-13, what="gates")
        _close(y, ref_y, 1e-12, what="layer y")


def pin_page_sizes(orc):
    """Record-size formula (nibbles + fp16 scale/bias per 64) against sizes on the pages."""
    with open(os.path.join(GOLDEN, "page_sizes.json")) as f:
        gold = json.load(f)
    rel = lambda a, b: abs(a - b) / b
    gem = orc.record_bytes(2816, 704)
    g = gold["gemma_expert_bytes"]
    assert rel(gem, g["value"]) <= g["rel_tol"], gem
    g = gold["gemma_installed_bytes"]
    total = g["layers"] * g["experts"] * gem + g["shared_core_bytes"]
    assert rel(total, g["value"]) <= g["rel_tol"], total
    glm_nib = 3 * 6144 * 2048 // 2
    g = gold["glm_expert_nibble_bytes"]
    assert rel(glm_nib, g["value"]) <= g["rel_tol"], glm_nib
    g = gold["glm_cold_token_bytes"]
    assert rel(g["layers"] * g["top_k"] * glm_nib, g["value"]) <= g["rel_tol"]


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
