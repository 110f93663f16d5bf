"""The sigmoid router (gate MOE_SIGMOID_TOPK) through the C ABI (needs a GPU).

Logistic scores, selection by score + per-expert bias, gates = routed_scale *
score / sum over the selection (the oracle's sigmoid_route).  Checked against
the oracle on the per-token path (1 and 3 tokens) and the grouped path
(9 and 40 tokens): ids bit-exact, gates within 1e-6 relative to the scale,
outputs within the usual 2e-3.  The bias is large enough to change the
selection: the tests count tokens whose biased selection differs from the
plain logit order.  The route call and the fused forward agree bit for bit.
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


@pytest.mark.parametrize("H,E,I,k,Is,T,scale,with_bias", [
    (256, 32, 128, 8, 256, 1, 2.5, True),
    (256, 32, 128, 8, 256, 3, 2.5, True),
    (320, 64, 192, 6, 0, 9, 1.0, True),
    (512, 256, 128, 8, 128, 40, 2.5, True),    # GLM-like expert count (4 key slots per lane)
    (256, 100, 128, 16, 128, 2, 1.8, False),   # no bias: the logit order
])
def test_sigmoid_router_matches_oracle(orc, H, E, I, k, Is, T, scale, with_bias):
    bias = None
    if with_bias:
        bias = np.random.default_rng(E + k).uniform(-0.15, 0.15, E).astype(np.float32)
    dl = DeviceLayer(0xB17E0800 + H + E + T, 0, H, E, I, k, Is, "bf16", gate="sigmoid",
                     routed_scale=scale, bias=bias)
    toks = [dl.natural_token(orc, s) for s in range(T)]
    x = to_dev(np.stack([t[0] for t in toks]), "bf16")
    ids, w, y = dl.layer_obj.forward(x)
    ids_r, w_r = dl.layer_obj.route(x)
    assert torch.equal(ids, ids_r) and torch.equal(w, w_r)
    ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
    worst_w = worst_y = 0.0
    moved = 0
    for t, (_, xd) in enumerate(toks):
        rid, rw, ry, _, _ = dl.oracle(orc, xd)
        assert ids[t].tolist() == rid.tolist(), f"token {t}: {ids[t]} vs {rid}"
        plain = orc.select_topk(orc.router_logits(dl.rq, dl.rs, xd), k)
        moved += int(plain.tolist() != rid.tolist())
        assert abs(float(np.sum(w[t])) - scale) <= 1e-5 * scale
        worst_w = max(worst_w, float(np.max(np.abs(w[t] - rw))))
        worst_y = max(worst_y, rel_err(y[t], ry))
    print(f"H{H} E{E} k{k} T{T} scale {scale}: {moved}/{T} selections moved by the bias; "
          f"max |w err| {worst_w:.2e}, max rel y err {worst_y:.2e}", flush=True)
    if with_bias:
        assert moved > 0
    assert worst_w <= W_TOL * scale and worst_y <= Y_TOL
