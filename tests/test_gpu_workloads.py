"""Full-size workloads on the GPU, checked against the oracle on sampled tokens.

* Gemma-4-A4B-scale stack: hidden 2816, 128 experts of intermediate 704, top-8,
  shared expert 2112, 30 layers (13.2 GB of records), bf16 activations, run
  through moe_stack_forward exactly as bench.py times it.
* GLM-scale decode: hidden 6144, 256 experts of intermediate 2048, top-8, shared
  2048 (5.5 GB per layer), activations drawn so the choice follows Zipf(1.1):
  4 layers x 8 steps through moe_stack_forward (per-token path), all 40 layers
  x 2 steps as bench.py holds them, and one call of 4 tokens (grouped path).
* GLM-scale 128-token prefill chunk (grouped path), 4-bit and 2-bit records.
The oracle regenerates the records it selects on the CPU from the seeded
generator; nothing the GPU computed is given to it.
"""
import numpy as np
import pytest
import torch

import synth
from _gpu_helpers import W_TOL, Y_TOL, DeviceLayer, elem_err, gap_ok, rel_err, to_dev, zipf_tokens
from bit_routed_expert_moe_amd import stack_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


@pytest.mark.timeout(900)
def test_gemma_stack_full_size(orc):
    """All 30 layers, 16 decode steps through moe_stack_forward: ids bit-exact,
    gates within 1e-6 and y within 2e-3 of the oracle on every token-layer (the
    oracle regenerates each selected record)."""
    wl = synth.WORKLOADS["gemma_a4b_h2816_e128_l30"]
    L, H, S = wl.n_layers, wl.hidden, 16
    layers = [DeviceLayer(wl.seed, l, H, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter, wl.act)
              for l in range(L)]
    ws = layers[0].layer_obj.workspace(1)
    worst_y = worst_w = 0.0
    for step in range(S):
        toks = [dl.natural_token(orc, step) for dl in layers]
        x = to_dev(np.stack([t[0] for t in toks])[:, None, :], wl.act)  # [L][1][H]
        ids, w, y = stack_forward([dl.layer_obj for dl in layers], x, ws)
        ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
        for l, dl in enumerate(layers):
            rid, rw, ry, _, _ = dl.oracle(orc, toks[l][1])
            worst_y = max(worst_y, rel_err(y[l, 0], ry))
            assert ids[l, 0].tolist() == rid.tolist(), f"step {step} layer {l}"
            worst_w = max(worst_w, float(np.max(np.abs(w[l, 0] - rw))))
    print(f"gemma stack: {S} steps x {L} layers, max |w err| {worst_w:.2e}, "
          f"max rel y err {worst_y:.2e}")
    assert worst_w <= W_TOL and worst_y <= Y_TOL


def test_glm_stack_decode_per_token(orc):
    """GLM-scale decode through the per-token path, as bench.py times it: 4
    layers of the 40-layer stack (hidden 6144, 256 experts of intermediate
    2048, top-8, shared 2048, bf16), Zipf(1.1) routing, 8 steps of one token
    each through moe_stack_forward (router launch, gate/up with in-launch
    top-k, down with the fixed-order combine: the 4-wave gate/up units and the
    down kernel's 8-groups-per-wave instance).  Then calls of 2 and 3 tokens on
    one layer, still the per-token path (fewer than 4 tokens).  ids bit-exact,
    gates within 1e-6, y within 2e-3 of the oracle on every token."""
    wl = synth.WORKLOADS["glm_h6144_e256_l40_zipf"]
    NL, S = 4, 8
    layers = [DeviceLayer(wl.seed, l, wl.hidden, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter, wl.act)
              for l in range(NL)]
    toks = [zipf_tokens(dl, orc, wl.zipf_s, range(S)) for dl in layers]  # [layer][step]
    ws = layers[0].layer_obj.workspace(1)
    worst_y = worst_w = worst_e = 0.0
    for step in range(S):
        x = to_dev(np.stack([toks[l][step][0] for l in range(NL)])[:, None, :], wl.act)  # [L][1][H]
        ids, w, y = stack_forward([dl.layer_obj for dl in layers], x, ws)
        ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
        for l, dl in enumerate(layers):
            rid, rw, ry, _, _ = dl.oracle(orc, toks[l][step][1])
            assert ids[l, 0].tolist() == rid.tolist(), f"step {step} layer {l}"
            worst_w = max(worst_w, float(np.max(np.abs(w[l, 0] - rw))))
            worst_y = max(worst_y, rel_err(y[l, 0], ry))
            worst_e = max(worst_e, elem_err(y[l, 0], ry))
    print(f"glm decode stack (T=1): {S} steps x {NL} layers, max |w err| {worst_w:.2e}, "
          f"max rel y err {worst_y:.2e}, element-wise (floor 1e-3 max|y|) {worst_e:.2e}", flush=True)
    assert worst_w <= W_TOL and worst_y <= Y_TOL
    dl = layers[1]
    for T in (2, 3):
        xq = np.stack([t[0] for t in toks[1][:T]])
        ids, w, y = dl.layer_obj.forward(to_dev(xq, wl.act))
        ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
        for t in range(T):
            rid, rw, ry, _, _ = dl.oracle(orc, toks[1][t][1])
            assert ids[t].tolist() == rid.tolist(), f"T={T} token {t}"
            assert np.max(np.abs(w[t] - rw)) <= W_TOL
            assert rel_err(y[t], ry) <= Y_TOL, f"T={T} token {t}: {rel_err(y[t], ry):.2e}"
        print(f"glm decode layer, T={T}: ok", flush=True)


@pytest.mark.timeout(900)
def test_glm_stack_all_40_layers(orc):
    """The GLM-scale stack exactly as bench.py holds it: all 40 layers (218 GB
    of records in HBM), Zipf(1.1) activations, 2 decode steps of one token
    through moe_stack_forward.  ids bit-exact and gates within 1e-6 on every
    layer of both steps; y within 2e-3 of the oracle on layers 0, 13, 26 and
    39 of the first step (the oracle regenerates each selected record)."""
    import gc
    wl = synth.WORKLOADS["glm_h6144_e256_l40_zipf"]
    NL, S = wl.n_layers, 2
    gc.collect()
    torch.cuda.empty_cache()  # room for 218 GB next to what earlier tests left cached
    layers = [DeviceLayer(wl.seed, l, wl.hidden, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter, wl.act)
              for l in range(NL)]
    print(f"glm stack: {NL} layers filled", flush=True)
    try:
        toks = [zipf_tokens(dl, orc, wl.zipf_s, range(S)) for dl in layers]
        ws = layers[0].layer_obj.workspace(1)
        worst_w = worst_y = 0.0
        for step in range(S):
            x = to_dev(np.stack([toks[l][step][0] for l in range(NL)])[:, None, :], wl.act)
            ids, w, y = stack_forward([dl.layer_obj for dl in layers], x, ws)
            ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
            for l, dl in enumerate(layers):
                xd = toks[l][step][1]
                if step == 0 and l in (0, 13, 26, 39):
                    rid, rw, ry, _, _ = dl.oracle(orc, xd)
                    worst_y = max(worst_y, rel_err(y[l, 0], ry))
                else:
                    rid, rw, _ = orc.route(dl.rq, dl.rs, xd, wl.top_k)
                assert ids[l, 0].tolist() == rid.tolist(), f"step {step} layer {l}"
                worst_w = max(worst_w, float(np.max(np.abs(w[l, 0] - rw))))
        print(f"glm stack, all {NL} layers: {S} steps, max |w err| {worst_w:.2e}, "
              f"max rel y err (sampled layers) {worst_y:.2e}", flush=True)
        assert worst_w <= W_TOL and worst_y <= Y_TOL
    finally:
        del layers
        gc.collect()
        torch.cuda.empty_cache()


def test_glm_layer_zipf_grouped_path(orc):
    """GLM-scale layer, 4 Zipf(1.1) tokens in one call: calls of 4 or more
    tokens take the grouped (expert-sorted MFMA) path.  ids bit-exact, gates
    within 1e-6, y within 2e-3 of the oracle."""
    wl = synth.WORKLOADS["glm_h6144_e256_l40_zipf"]
    dl = DeviceLayer(wl.seed, 0, wl.hidden, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter, wl.act)
    toks = zipf_tokens(dl, orc, wl.zipf_s, range(4))
    ids, w, y = dl.layer_obj.forward(to_dev(np.stack([t[0] for t in toks]), wl.act))
    ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
    worst = 0.0
    for t, (_, xd) in enumerate(toks):
        rid, rw, ry, _, _ = dl.oracle(orc, xd)
        assert ids[t].tolist() == rid.tolist()
        assert np.max(np.abs(w[t] - rw)) <= W_TOL
        worst = max(worst, rel_err(y[t], ry))
    print(f"glm zipf layer, grouped path: {len(toks)} tokens, max rel y err {worst:.2e}")
    assert worst <= Y_TOL


@pytest.mark.timeout(900)
@pytest.mark.parametrize("bits", [4, 2])
def test_glm_prefill_chunk_full_size(orc, bits):
    """GLM-scale 128-token chunk (uniform random routing realised through the
    router) through the grouped path: every token's ids, gate weights and
    output against the oracle (which regenerates each selected record on the
    CPU), and the whole chunk's result permuted exactly with its tokens.
    4-bit and 2-bit records."""
    wl = synth.WORKLOADS["glm_prefill_h6144_e256_t128"]
    dl = DeviceLayer(wl.seed, 0, wl.hidden, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter, wl.act,
                     bits=bits)
    Wd = dl.rq.astype(np.float64) * dl.rs.view(np.float16).astype(np.float64)[:, None]
    zr = synth.ZipfRealiser(Wd, wl.zipf_s, wl.seed, 0)  # s = 0: uniform Gumbel-top-8 targets
    toks = []
    for t in range(wl.n_tokens):
        for a in range(50):
            xq = synth.quantize_act(zr.activations(t, a)[0], wl.act)
            xd = orc.act_to_f64(wl.act, xq)
            if gap_ok(orc.router_logits(dl.rq, dl.rs, xd), wl.top_k):
                break
        toks.append((xq, xd))
    n_unique = len({int(e) for t in toks for e in orc.route(dl.rq, dl.rs, t[1], wl.top_k)[0]})
    print(f"glm prefill chunk: {n_unique} distinct experts selected", flush=True)
    assert n_unique > 230  # uniform: 256 * (1 - (1 - 8/256)^128) = 251.6 expected
    xq = np.stack([t[0] for t in toks])
    ws = dl.layer_obj.workspace(wl.n_tokens)
    ids, w, y = dl.layer_obj.forward(to_dev(xq, wl.act), ws)
    ids_h, w_h, y_h = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
    worst_w = 0.0
    for t, (_, xd) in enumerate(toks):
        rid, rw, _ = orc.route(dl.rq, dl.rs, xd, wl.top_k)
        assert ids_h[t].tolist() == rid.tolist(), f"token {t}"
        worst_w = max(worst_w, float(np.max(np.abs(w_h[t] - rw))))
    assert worst_w <= W_TOL
    worst_y = 0.0
    for t in range(wl.n_tokens):
        _, _, ry, _, _ = dl.oracle(orc, toks[t][1])
        worst_y = max(worst_y, rel_err(y_h[t], ry))
        if t % 32 == 31:
            print(f"glm prefill tokens 0..{t}: max rel y err {worst_y:.2e}", flush=True)
    print(f"{bits}-bit glm prefill chunk: {wl.n_tokens} tokens, max |w err| {worst_w:.2e}, "
          f"max rel y err {worst_y:.2e}")
    assert worst_y <= Y_TOL
    perm = np.random.default_rng(2).permutation(wl.n_tokens)
    ids2, w2, y2 = dl.layer_obj.forward(to_dev(xq[perm], wl.act), ws)
    p = torch.from_numpy(perm).cuda()
    assert torch.equal(ids[p], ids2) and torch.equal(w[p], w2) and torch.equal(y[p], y2)
