"""Routing inside the gate/up launch (the resident forward) through the C ABI
(needs a GPU).

The resident forward computes the router logits in leading workgroups of the
gate/up launch; the gate/up workgroups read them as they land and, after a
bounded number of polls, compute them locally instead (above hidden 4096 a
separate router launch runs first, and the limit changes nothing).  A layer created with
MOE_ROUTE_SPIN_LIMIT=-1 always computes them locally and one created with 0
polls once: both must give the default layer's ids, gates and outputs bit for
bit, and the oracle's selection.  The logit words go back to zero after every
call (a later call would otherwise select from stale logits): a sequence of
different tokens on one workspace gives what fresh workspaces give, also
when layers of different shapes take turns on it.
"""
import numpy as np
import pytest
import torch

from _gpu_helpers import W_TOL, Y_TOL, DeviceLayer, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def twin(dl, monkeypatch, limit):
    """The same weights in a layer created under MOE_ROUTE_SPIN_LIMIT=limit."""
    from bit_routed_expert_moe_amd import Layer
    monkeypatch.setenv("MOE_ROUTE_SPIN_LIMIT", str(limit))
    try:
        return Layer(dl.H, dl.E, dl.I, dl.k, dl.Is, torch.from_numpy(dl.rq).cuda(),
                     torch.from_numpy(dl.rs.view(np.float16)).cuda(), dl.pool, dl.shared, act=dl.act,
                     gate=dl.gate, routed_scale=dl.routed_scale, selection_bias=dl.bias_dev,
                     bits=dl.bits)
    finally:
        monkeypatch.delenv("MOE_ROUTE_SPIN_LIMIT")


CASES = [
    # H, E, I, k, Is, T, act, gate, bits
    (256, 32, 128, 8, 256, 1, "bf16", "softmax", 4),
    (512, 64, 192, 6, 320, 3, "f32", "softmax", 4),     # 3 tokens, fp32 activations
    (2816, 128, 704, 8, 2112, 1, "bf16", "softmax", 4),  # Gemma-scale shapes
    (768, 256, 128, 8, 128, 2, "bf16", "sigmoid", 4),   # sigmoid gate with bias, 4 key slots
    (5120, 200, 128, 8, 128, 1, "bf16", "softmax", 4),  # hidden > 4096: separate router launch
    (5120, 200, 128, 8, 128, 1, "bf16", "softmax", 2),  # the same with 2-bit records
    (4608, 72, 128, 8, 128, 2, "f32", "softmax", 4),    # hidden > 4096, fp32 activations, 2 tokens
    (8192, 16, 64, 2, 128, 1, "bf16", "softmax", 4),    # largest hidden, few experts
    (1024, 1024, 64, 16, 0, 1, "f32", "softmax", 2),   # most experts, largest k, 2-bit
    (192, 7, 64, 3, 0, 2, "bf16", "softmax", 2),       # fewer experts than waves
]


@pytest.mark.parametrize("H,E,I,k,Is,T,act,gate,bits", CASES)
def test_local_logits_give_the_same_bits(orc, monkeypatch, H, E, I, k, Is, T, act, gate, bits):
    bias = (np.random.default_rng(E).uniform(-0.15, 0.15, E).astype(np.float32)
            if gate == "sigmoid" else None)
    dl = DeviceLayer(0xF05E0000 + H + E + T, 0, H, E, I, k, Is, act, gate=gate,
                     routed_scale=2.5 if gate == "sigmoid" else 1.0, bias=bias, bits=bits)
    toks = [dl.natural_token(orc, s) for s in range(T)]
    x = to_dev(np.stack([t[0] for t in toks]), act)
    ref = dl.layer_obj.forward(x)
    ids = ref[0].cpu().numpy()
    for t, (_, xd) in enumerate(toks):
        rid, rw, ry, _, _ = dl.oracle(orc, xd)
        assert ids[t].tolist() == rid.tolist(), f"token {t}"
        assert np.max(np.abs(ref[1].cpu().numpy()[t] - rw)) <= W_TOL * dl.routed_scale
        assert rel_err(ref[2].cpu().numpy()[t], ry) <= Y_TOL
    for limit in (-1, 0):
        got = twin(dl, monkeypatch, limit).forward(x)
        for a_, b_ in zip(ref, got):
            assert torch.equal(a_, b_), f"spin limit {limit}: result differs from the default"


def test_logit_words_return_to_zero_between_calls(orc):
    """Different tokens one after another on one workspace, each equal to the
    same call on a fresh zero-filled workspace."""
    dl = DeviceLayer(0xF05E0100, 0, 512, 48, 192, 8, 256, "bf16")
    ws = dl.layer_obj.workspace(3)
    for step in range(8):
        T = 1 + step % 3
        toks = [dl.natural_token(orc, 3 * step + t) for t in range(T)]
        x = to_dev(np.stack([t[0] for t in toks]), "bf16")
        shared_ws = dl.layer_obj.forward(x, ws)
        fresh = dl.layer_obj.forward(x, dl.layer_obj.workspace(T))
        for a_, b_ in zip(shared_ws, fresh):
            assert torch.equal(a_, b_), f"step {step}: reused workspace differs"
        for t, (_, xd) in enumerate(toks):
            assert shared_ws[0].cpu().numpy()[t].tolist() == dl.oracle(orc, xd)[0].tolist()


def test_layers_of_different_shapes_share_one_workspace(orc):
    """Layers of three shapes take turns on one workspace sized for the largest;
    each call equals the same call on a fresh zero-filled workspace (the
    arrival counters and logit words sit at the same offsets, with the same
    extents, for every shape)."""
    shapes = [(512, 48, 192, 8, 256, "bf16"), (4096, 200, 128, 6, 128, "f32"), (256, 16, 64, 4, 0, "bf16"),
              (6144, 64, 128, 8, 128, "bf16")]
    dls = [DeviceLayer(0xF05E0200 + i, 0, H, E, I, k, Is, act) for i, (H, E, I, k, Is, act) in enumerate(shapes)]
    nbytes = max(dl.layer_obj.workspace_bytes(3) for dl in dls)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for step in range(12):
        dl = dls[step % len(dls)]
        T = 1 + step % 3
        toks = [dl.natural_token(orc, 3 * step + t) for t in range(T)]
        x = to_dev(np.stack([t[0] for t in toks]), dl.act)
        got = dl.layer_obj.forward(x, ws)
        fresh = dl.layer_obj.forward(x, dl.layer_obj.workspace(T))
        for a_, b_ in zip(got, fresh):
            assert torch.equal(a_, b_), f"step {step} (H {dl.H}, E {dl.E}, T {T}): shared workspace differs"
        for t, (_, xd) in enumerate(toks):
            assert got[0].cpu().numpy()[t].tolist() == dl.oracle(orc, xd)[0].tolist()
