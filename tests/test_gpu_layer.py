"""Parity of the HIP path against the CPU oracle, through the C ABI (needs a GPU).

Bar: expert ids bit-exact (tokens are drawn so the oracle's top-(k+1) logits
are separated by more than 1e-4), gate weights within 1e-6, outputs within a
max relative error of 2e-3 per token (max |y - y_ref| / max |y_ref|).
Special cases with closed forms: one dominant expert (a dense SwiGLU),
constant weights, zero scales (bias terms only), integer activations (exact
logits, ties included).
"""
import sys

import numpy as np
import pytest
import torch

import synth
import synth.gpu
from _gpu_helpers import W_TOL, Y_TOL, DeviceLayer, elem_err, rel_err, to_dev
from _packer import DenseExpert

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def check_tokens(dl, orc, xs_q, xs_d, ids, w, y, tag):
    worst_y, worst_w, worst_e = 0.0, 0.0, 0.0
    for t in range(len(xs_d)):
        rid, rw, ry, _, _ = dl.oracle(orc, xs_d[t])
        assert ids[t].tolist() == rid.tolist(), f"{tag} token {t}: ids {ids[t]} vs {rid}"
        worst_w = max(worst_w, float(np.max(np.abs(w[t] - rw))))
        worst_y = max(worst_y, rel_err(y[t], ry))
        worst_e = max(worst_e, elem_err(y[t], ry))
    say(f"{tag}: {len(xs_d)} tokens, max |w err| {worst_w:.2e}, max rel y err {worst_y:.2e}, "
        f"element-wise (floor 1e-3 max|y|) {worst_e:.2e}")
    assert worst_w <= W_TOL and worst_y <= Y_TOL


@pytest.mark.parametrize("bits", [4, 2])
def test_gpu_fill_matches_cpu_generator(bits):
    for H, I, first, n in [(256, 128, 0, 3), (2816, 704, 5, 2), (64, 64, -1, 1)]:
        rb = synth.record_bytes(H, I, bits)
        buf = torch.empty(rb * n, dtype=torch.uint8, device="cuda")
        synth.gpu.fill_records(buf, H, I, 77, 3, first, n, bits=bits)
        got = buf.cpu().numpy()
        for r in range(n):
            e = synth.SHARED_INDEX if first < 0 else first + r
            assert np.array_equal(got[r * rb:(r + 1) * rb], synth.expert_record(77, 3, e, H, I, bits))


def test_tiny_layer_many_tokens(orc):
    """The tiny fp32 layer on 192 separated tokens, as one batch and one by one."""
    wl = synth.WORKLOADS["tiny_h256_e32"]
    dl = DeviceLayer(wl.seed, 0, wl.hidden, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter, wl.act)
    toks = [dl.natural_token(orc, s) for s in range(192)]
    xq = np.stack([t[0] for t in toks]); xd = [t[1] for t in toks]
    ids, w, y = dl.layer_obj.forward(to_dev(xq, wl.act))
    check_tokens(dl, orc, xq, xd, ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy(), "tiny T=192")
    # batches of 4 or more tokens take the grouped path, smaller ones the decode
    # path: within a path a token's result does not depend on its batch
    i8, w8, y8 = dl.layer_obj.forward(to_dev(xq[100:108], wl.act))
    assert torch.equal(i8, ids[100:108]) and torch.equal(y8, y[100:108]), \
        "a token's result depends on the batch"
    i2, _, y2 = dl.layer_obj.forward(to_dev(xq[:2], wl.act))
    for t in range(2):
        i1, _, y1 = dl.layer_obj.forward(to_dev(xq[t:t + 1], wl.act))
        assert torch.equal(i1[0], i2[t]) and torch.equal(y1[0], y2[t])
    check_tokens(dl, orc, xq[:2], xd[:2], i2.cpu().numpy(), w[:2].cpu().numpy(),
                 y2.cpu().numpy(), "tiny T=2 (decode path)")


@pytest.mark.parametrize("H,E,I,k,Is,T", [
    (512, 40, 192, 6, 320, 24),     # grouped path
    (512, 40, 192, 6, 320, 1),      # per-token: separate kernels vs the one-launch FFN (routing inside)
    (512, 40, 192, 6, 320, 3),
    (4608, 72, 1024, 8, 1024, 1),   # per-token above hidden 4096 (router launch, then the FFN launch)
    (4608, 72, 1024, 8, 1024, 3),
])
def test_api_calls_match_fused_forward_bitwise(orc, H, E, I, k, Is, T):
    """route -> expert_ffn -> combine gives exactly the fused forward's result,
    and each per-expert output matches the oracle's expert.  On the per-token
    path the API calls run the gate/up and down kernels as two launches and
    the forward runs them as one."""
    dl = DeviceLayer(0xB17E0101, 0, H, E, I, k, Is, "bf16")
    toks = [dl.natural_token(orc, s) for s in range(T)]
    x = to_dev(np.stack([t[0] for t in toks]), "bf16")
    ws = dl.layer_obj.workspace(x.shape[0])
    ids_f, w_f, y_f = dl.layer_obj.forward(x, ws)
    ids_r, w_r = dl.layer_obj.route(x, ws)
    eo = dl.layer_obj.ffn(x, ids_r, ws)
    y_c = dl.layer_obj.combine(eo, w_r)
    assert torch.equal(ids_f, ids_r) and torch.equal(w_f, w_r)
    assert torch.equal(y_f, y_c)
    eo = eo.cpu().numpy()
    for t, (_, xd) in enumerate(toks):
        rid, rw, ry, yr, ys = dl.oracle(orc, xd)
        for j in range(dl.k):
            assert rel_err(eo[t, j], yr[j]) <= Y_TOL
        assert rel_err(eo[t, dl.k], ys) <= Y_TOL
    yb = dl.layer_obj.combine(torch.from_numpy(eo).cuda(), w_r, torch.bfloat16)
    ref = torch.from_numpy(y_c.cpu().numpy()).to(torch.bfloat16)
    assert torch.equal(yb.cpu(), ref), "bf16 output is not the nearest-even rounding"


SHAPES = [
    (192, 7, 64, 3, 0, "bf16"),        # fewer input groups than waves, no shared expert
    (320, 64, 192, 8, 320, "bf16"),    # ragged splits everywhere
    (64, 1, 64, 1, 64, "f32"),         # minimum sizes, a single expert
    (1024, 1024, 128, 16, 0, "bf16"),  # most experts, largest k
    (8192, 16, 64, 2, 128, "bf16"),    # largest hidden
    (2816, 128, 704, 8, 2112, "f32"),  # Gemma-scale shapes with fp32 activations
    (4160, 32, 1152, 8, 640, "bf16"),  # 4-wave gate/up with a ragged last wave; 5 down groups per wave
    (2048, 96, 2048, 8, 2048, "f32"),  # intermediate 2048 (8 down groups per wave), fp32
    (8192, 64, 4096, 4, 0, "bf16"),    # largest hidden and intermediate: 32 gate/up and 16 down groups per wave
]


@pytest.mark.parametrize("T", [1, 3, 6])
@pytest.mark.parametrize("H,E,I,k,Is,act", SHAPES)
def test_shapes(orc, H, E, I, k, Is, act, T):
    """Each shape through one call of T tokens: T = 1 and 3 take the per-token
    (decode) kernels, T = 6 the grouped path.  ids bit-exact, gates within
    1e-6, y within 2e-3 of the oracle on every token."""
    dl = DeviceLayer(0xB17E0200 + H + E, 1, H, E, I, k, Is, act)
    toks = [dl.natural_token(orc, s) for s in range(T)]
    xq = np.stack([t[0] for t in toks])
    ids, w, y = dl.layer_obj.forward(to_dev(xq, act))
    path = "grouped" if T >= 4 else "per-token"
    check_tokens(dl, orc, xq, [t[1] for t in toks], ids.cpu().numpy(), w.cpu().numpy(),
                 y.cpu().numpy(), f"H{H} E{E} I{I} k{k} S{Is} {act} T={T} ({path})")


def test_dense_swiglu_special_case():
    """k = 1 with one dominant expert and no shared expert reproduces a dense
    SwiGLU computed with library matmuls on the dequantised matrices."""
    from bit_routed_expert_moe_amd import Layer
    rng = np.random.default_rng(5)
    H, I, E = 256, 192, 3
    exps = [DenseExpert(H, I, rng) for _ in range(E)]
    pool = torch.from_numpy(np.concatenate([e.rec for e in exps])).cuda()
    rq = np.zeros((E, H), dtype=np.int8); rq[2, :] = 1
    rs = np.ones(E, dtype=np.float16)
    lay = Layer(H, E, I, 1, 0, torch.from_numpy(rq).cuda(), torch.from_numpy(rs).cuda(), pool,
                None, act="f32")
    for _ in range(4):
        x = np.abs(rng.standard_normal(H)).astype(np.float32)
        ids, w, y = lay.forward(torch.from_numpy(x[None]).cuda())
        assert ids.item() == 2 and w.item() == 1.0
        assert rel_err(y.cpu().numpy()[0], exps[2].ffn(x.astype(np.float64))) <= Y_TOL


def test_constant_weights_closed_form():
    """Constant nibbles/scales/biases: y_o = (s'c'+b') * I * silu(gamma) * gamma,
    gamma = (s c + b) * sum(x)."""
    from bit_routed_expert_moe_amd import Layer
    rng = np.random.default_rng(6)
    H, I = 512, 128
    c, s, b, c2, s2, b2 = 5, 2.0 ** -7, -(2.0 ** -9), 9, 2.0 ** -8, 2.0 ** -10
    f16 = lambda v, shape: np.full(shape, np.float16(v)).view(np.uint16)
    ex = DenseExpert(H, I, rng, qG=np.full((I, H), c), qU=np.full((I, H), c), qD=np.full((H, I), c2),
                     sb=(f16(s, (I, H // 64)), f16(b, (I, H // 64)), f16(s, (I, H // 64)),
                         f16(b, (I, H // 64)), f16(s2, (H, I // 64)), f16(b2, (H, I // 64))))
    lay = Layer(H, 1, I, 1, 0, torch.zeros(1, H, dtype=torch.int8).cuda(),
                torch.ones(1, dtype=torch.float16).cuda(), torch.from_numpy(ex.rec).cuda(), None,
                act="f32")
    x = rng.standard_normal(H).astype(np.float32)
    gamma = (s * c + b) * float(x.astype(np.float64).sum())
    yref = (s2 * c2 + b2) * I * gamma / (1 + np.exp(-gamma)) * gamma
    _, _, y = lay.forward(torch.from_numpy(x[None]).cuda())
    assert rel_err(y.cpu().numpy()[0], np.full(H, yref)) <= Y_TOL


@pytest.mark.parametrize("bits", [4, 2])
def test_zero_scales_leave_the_bias_terms(bits):
    """Every scale 0: W = bias per group, whatever the codes, so the output is
    the dense SwiGLU of the bias-only matrices (the code products must vanish
    and the bias * sum(x) terms carry everything)."""
    from bit_routed_expert_moe_amd import Layer
    rng = np.random.default_rng(8)
    H, I = 320, 192
    z = lambda shape: np.zeros(shape, dtype=np.uint16)  # fp16 +0
    f16 = lambda shape: rng.uniform(-8e-3, 8e-3, shape).astype(np.float16).view(np.uint16)
    ex = DenseExpert(H, I, rng, sb=(z((I, H // 64)), f16((I, H // 64)), z((I, H // 64)),
                                    f16((I, H // 64)), z((H, I // 64)), f16((H, I // 64))), bits=bits)
    assert not np.any(ex.G - np.repeat(ex.G[:, ::64], 64, axis=1))  # bias-only, constant per group
    lay = Layer(H, 1, I, 1, 0, torch.zeros(1, H, dtype=torch.int8).cuda(),
                torch.ones(1, dtype=torch.float16).cuda(), torch.from_numpy(ex.rec).cuda(), None,
                act="f32", bits=bits)
    for _ in range(3):
        x = rng.standard_normal(H).astype(np.float32)
        _, _, y = lay.forward(torch.from_numpy(x[None]).cuda())
        assert rel_err(y.cpu().numpy()[0], ex.ffn(x.astype(np.float64))) <= Y_TOL


def test_integer_activations_give_exact_logits():
    """Integer activations make every router logit an exact integer times the
    row scale (all products and partial sums are exact in fp32), ties included:
    ids must follow (logit descending, lower id first) exactly and the gates
    are the softmax of those exact logits."""
    from bit_routed_expert_moe_amd import Layer
    rng = np.random.default_rng(9)
    H, E, I, k = 256, 48, 64, 8
    rq = rng.integers(-3, 4, (E, H)).astype(np.int8)
    rq[7] = rq[3]  # an exact tie between experts 3 and 7
    rs = np.full(E, 1.0 / 256, dtype=np.float16)
    pool = torch.zeros(E * DenseExpert(H, I, rng).rec.size, dtype=torch.uint8).cuda()
    lay = Layer(H, E, I, k, 0, torch.from_numpy(rq).cuda(), torch.from_numpy(rs).cuda(), pool, None,
                act="f32")
    for trial in range(4):
        x = rng.integers(-4, 5, H).astype(np.float32)
        ids, w = lay.route(torch.from_numpy(x[None]).cuda())
        exact = (rq.astype(np.int64) @ x.astype(np.int64)).astype(np.float64) / 256.0
        order = sorted(range(E), key=lambda e: (-exact[e], e))[:k]
        assert ids.cpu().numpy()[0].tolist() == order, trial
        sel = exact[order]
        wref = np.exp(sel - sel.max()) / np.exp(sel - sel.max()).sum()
        assert np.max(np.abs(w.cpu().numpy()[0] - wref)) <= W_TOL


@pytest.mark.parametrize("T", [1, 3, 4])
def test_rerun_is_bitwise_identical(orc, T):
    """Two calls on one workspace and one on a fresh workspace give the same
    bits: T = 1 and 3 on the per-token path, T = 4 on the grouped path."""
    dl = DeviceLayer(0xB17E0300, 0, 2816, 128, 704, 8, 2112, "bf16")
    toks = [dl.natural_token(orc, s) for s in range(T)]
    x = to_dev(np.stack([t[0] for t in toks]), "bf16")
    ws = dl.layer_obj.workspace(T)
    r1 = dl.layer_obj.forward(x, ws)
    r2 = dl.layer_obj.forward(x, ws)
    r3 = dl.layer_obj.forward(x)  # fresh workspace
    for a, b, c in zip(r1, r2, r3):
        assert torch.equal(a, b) and torch.equal(a, c)


def test_bad_ids_raise_device_error_and_poison():
    from bit_routed_expert_moe_amd import MoeError
    dl = DeviceLayer(0xB17E0400, 0, 256, 16, 128, 4, 128, "bf16")
    x = to_dev(synth.quantize_act(synth.activations(1, 0, 0, 256, n_tokens=2), "bf16"), "bf16")
    ws = dl.layer_obj.workspace(2)
    dl.layer_obj.poll_error(ws)
    ids = torch.tensor([[0, 1, 16, 3], [4, -1, 6, 7]], dtype=torch.int32, device="cuda")
    eo = dl.layer_obj.ffn(x, ids, ws).cpu().numpy()
    with pytest.raises(MoeError) as ei:
        dl.layer_obj.poll_error(ws)
    assert ei.value.status == -8
    dl.layer_obj.poll_error(ws)  # cleared
    assert np.all(np.isnan(eo[0, 2])) and np.all(np.isnan(eo[1, 1]))
    good = [(0, 0), (0, 1), (0, 3), (0, 4), (1, 0), (1, 2), (1, 3), (1, 4)]
    for t, j in good:
        assert np.all(np.isfinite(eo[t, j]))
