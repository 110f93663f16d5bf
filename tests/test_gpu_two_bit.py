"""2-bit expert records (desc.bits = 2) through the C ABI (needs a GPU).

The affine group-64 format with 2-bit codes, checked against the oracle's
expert FFN on the same records (bits=2) and the oracle's routing: ids
bit-exact, gates within 1e-6, outputs within the usual 2e-3 relative per token.
Calls of 4 or more tokens take the grouped (MFMA) path, where a token's
result does not depend on the rest of its batch.  The three-call API agrees
with the fused forward bit for bit, a slot-cached 2-bit layer agrees with the
resident one, the Gemma-scale stack (30 layers, the shape and the call the
benchmark times) is checked on two decode steps of every layer, and so is
GLM-scale decode on two layers.  More grouped shapes run 2-bit records in the
prefill tests.
"""
import numpy as np
import pytest
import torch

import synth
from _gpu_helpers import W_TOL, Y_TOL, DeviceLayer, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def check(dl, orc, toks, ids, w, y, tag):
    ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
    worst_w = worst_y = 0.0
    for t, (_, xd) in enumerate(toks):
        rid, rw, ry, _, _ = dl.oracle(orc, xd)
        assert ids[t].tolist() == rid.tolist(), f"{tag} token {t}: {ids[t]} vs {rid}"
        worst_w = max(worst_w, float(np.max(np.abs(w[t] - rw))))
        worst_y = max(worst_y, rel_err(y[t], ry))
    print(f"{tag}: {len(toks)} tokens, max |w err| {worst_w:.2e}, max rel y err {worst_y:.2e}",
          flush=True)
    assert worst_w <= W_TOL * dl.routed_scale and worst_y <= Y_TOL


@pytest.mark.parametrize("H,E,I,k,Is,T,act", [
    (256, 32, 128, 8, 256, 1, "f32"),
    (256, 32, 128, 8, 256, 3, "bf16"),
    (320, 64, 192, 6, 320, 7, "bf16"),    # grouped path, ragged splits
    (192, 7, 64, 3, 0, 2, "bf16"),        # fewer input groups than waves, no shared expert
    (64, 1, 64, 1, 64, 1, "f32"),         # minimum sizes, a single expert
    (1024, 1024, 128, 16, 0, 1, "bf16"),  # most experts, largest k
    (8192, 16, 64, 2, 128, 1, "bf16"),    # largest hidden
    (2816, 128, 704, 8, 2112, 5, "f32"),  # Gemma-scale shapes, fp32 activations, grouped
])
def test_two_bit_matches_oracle(orc, H, E, I, k, Is, T, act):
    dl = DeviceLayer(0xB17E2B00 + H + E + T, 0, H, E, I, k, Is, act, bits=2)
    toks = [dl.natural_token(orc, s) for s in range(T)]
    xq = np.stack([t[0] for t in toks])
    ids, w, y = dl.layer_obj.forward(to_dev(xq, act))
    check(dl, orc, toks, ids, w, y, f"2-bit H{H} E{E} I{I} k{k} Is{Is} T{T} {act}")
    if T >= 5:  # a 4-token sub-batch (also grouped) gives exactly its rows of the batch
        i4, w4, y4 = dl.layer_obj.forward(to_dev(xq[1:5], act))
        assert torch.equal(i4, ids[1:5]) and torch.equal(w4, w[1:5]) and torch.equal(y4, y[1:5])


def test_two_bit_sigmoid_router(orc):
    E = 256
    bias = np.random.default_rng(E).uniform(-0.15, 0.15, E).astype(np.float32)
    dl = DeviceLayer(0xB17E2B10, 0, 512, E, 128, 8, 128, "bf16", gate="sigmoid",
                     routed_scale=2.5, bias=bias, bits=2)
    toks = [dl.natural_token(orc, s) for s in range(6)]
    ids, w, y = dl.layer_obj.forward(to_dev(np.stack([t[0] for t in toks]), "bf16"))
    check(dl, orc, toks, ids, w, y, "2-bit sigmoid E256")


def test_two_bit_api_calls_match_fused_forward_bitwise(orc):
    """route -> expert_ffn -> combine on 3 tokens (per-token path) gives exactly
    the fused forward's result; each per-expert output matches the oracle's."""
    dl = DeviceLayer(0xB17E2B20, 0, 512, 40, 192, 6, 320, "bf16", bits=2)
    toks = [dl.natural_token(orc, s) for s in range(3)]
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
        _, _, _, yr, ys = dl.oracle(orc, xd)
        for j in range(dl.k):
            assert rel_err(eo[t, j], yr[j]) <= Y_TOL
        assert rel_err(eo[t, dl.k], ys) <= Y_TOL


def test_two_bit_slot_cache_matches_resident(orc):
    from bit_routed_expert_moe_amd import Layer, record_bytes
    H, E, I, k, Is, n_slots = 512, 48, 192, 8, 256, 12
    dl = DeviceLayer(0xB17E2B40, 0, H, E, I, k, Is, "bf16", bits=2)
    host = torch.empty(dl.pool.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(dl.pool.cpu())
    slots = torch.zeros(n_slots * record_bytes(H, I, 2), dtype=torch.uint8, device="cuda")
    cached = Layer(H, E, I, k, Is, torch.from_numpy(dl.rq).cuda(),
                   torch.from_numpy(dl.rs.view(np.float16)).cuda(), None, dl.shared, act="bf16",
                   n_slots=n_slots, host_pool=host, slots=slots, bits=2)
    ws_r, ws_c = dl.layer_obj.workspace(1), cached.workspace(1)
    for step in range(16):
        xq, xd = dl.natural_token(orc, step)
        x = to_dev(xq[None], "bf16")
        r = dl.layer_obj.forward(x, ws_r)
        c = cached.forward(x, ws_c)
        for a_, b_ in zip(r, c):
            assert torch.equal(a_, b_), f"step {step}: cached result differs from resident"
        if step < 2:
            check(dl, orc, [(xq, xd)], *r, f"2-bit cached step {step}")
    hits, misses = cached.cache_stats()
    assert hits + misses == 16 * k and misses >= n_slots


def test_two_bit_gemma_stack_full_size(orc):
    """The Gemma-scale stack of 2-bit layers through moe_stack_forward (one token
    per layer, as timed): 30 layers x 128 records of 1.86 MB."""
    from bit_routed_expert_moe_amd import stack_forward
    wl = synth.WORKLOADS["gemma_a4b_h2816_e128_l30"]
    L, H = wl.n_layers, wl.hidden
    layers = [DeviceLayer(wl.seed, l, H, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter, wl.act,
                          bits=2) for l in range(L)]
    ws = layers[0].layer_obj.workspace(1)
    worst_y = worst_w = 0.0
    for step in range(2):
        toks = [dl.natural_token(orc, step) for dl in layers]
        x = to_dev(np.stack([t[0] for t in toks])[:, None, :], wl.act)
        ids, w, y = stack_forward([dl.layer_obj for dl in layers], x, ws)
        ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
        for l, dl in enumerate(layers):
            rid, rw, ry, _, _ = dl.oracle(orc, toks[l][1])
            assert ids[l, 0].tolist() == rid.tolist(), f"step {step} layer {l}"
            worst_w = max(worst_w, float(np.max(np.abs(w[l, 0] - rw))))
            worst_y = max(worst_y, rel_err(y[l, 0], ry))
    print(f"2-bit gemma stack: 2 steps x {L} layers, max |w err| {worst_w:.2e}, "
          f"max rel y err {worst_y:.2e}", flush=True)
    assert worst_w <= W_TOL and worst_y <= Y_TOL


def test_two_bit_glm_decode(orc):
    """GLM-scale decode with 2-bit records (the bench's --bits 2 line): hidden
    6144 (4-wave gate/up units, the shared expert in quarters of H), 256
    experts of intermediate 2048, shared 2048, Zipf(1.1) activations; 2 layers
    x 4 steps of one token through moe_stack_forward, then a 3-token call on
    one layer (still the per-token path)."""
    from _gpu_helpers import zipf_tokens
    from bit_routed_expert_moe_amd import stack_forward
    wl = synth.WORKLOADS["glm_h6144_e256_l40_zipf"]
    NL, S = 2, 4
    layers = [DeviceLayer(wl.seed, l, wl.hidden, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter, wl.act,
                          bits=2) for l in range(NL)]
    toks = [zipf_tokens(dl, orc, wl.zipf_s, range(S)) for dl in layers]
    ws = layers[0].layer_obj.workspace(1)
    for step in range(S):
        x = to_dev(np.stack([toks[l][step][0] for l in range(NL)])[:, None, :], wl.act)
        ids, w, y = stack_forward([dl.layer_obj for dl in layers], x, ws)
        for l, dl in enumerate(layers):
            check(dl, orc, [toks[l][step]], ids[l], w[l], y[l], f"2-bit glm decode step {step} layer {l}")
    dl = layers[0]
    ids, w, y = dl.layer_obj.forward(to_dev(np.stack([t[0] for t in toks[0][:3]]), wl.act))
    check(dl, orc, toks[0][:3], ids, w, y, "2-bit glm decode, 3 tokens")
