"""The multi-token (grouped, MFMA) path through the C ABI (needs a GPU).

Calls with 4 or more tokens sort the (token, slot) pairs by expert and run each
selected expert once over all of its tokens.  Checked here:

* ids bit-exact, gate weights within 1e-6 and outputs within a max relative
  error of 2e-3 per token against the oracle, on ragged shapes (tokens not a
  multiple of the 16-row tile, hidden sizes whose 32-input chunks do not split
  evenly over four waves, shared expert wider, narrower or absent, one expert
  taking every token, up to 1024 experts and k = 16);
* per-slot expert outputs of moe_expert_ffn against the oracle's experts, and
  route -> expert_ffn -> combine equal to the fused forward bit for bit;
* a token's result does not depend on the other tokens of its batch
  (permuting the batch permutes the result exactly);
* out-of-range expert ids raise the device error and poison only their slots.
Shapes, the API path and the batch invariance run for 4-bit and 2-bit records.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from _gpu_helpers import W_TOL, Y_TOL, DeviceLayer, rel_err, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def tokens(dl, orc, n, first=0):
    toks = [dl.natural_token(orc, first + s) for s in range(n)]
    return np.stack([t[0] for t in toks]), [t[1] for t in toks]


def check(dl, orc, xd, ids, w, y, tag, sample=None):
    ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
    worst_w = worst_y = 0.0
    for t in (range(len(xd)) if sample is None else sample):
        rid, rw, ry, _, _ = dl.oracle(orc, xd[t])
        assert ids[t].tolist() == rid.tolist(), f"{tag} token {t}: ids {ids[t]} vs {rid}"
        worst_w = max(worst_w, float(np.max(np.abs(w[t] - rw))))
        worst_y = max(worst_y, rel_err(y[t], ry))
    say(f"{tag}: max |w err| {worst_w:.2e}, max rel y err {worst_y:.2e}")
    assert worst_w <= W_TOL and worst_y <= Y_TOL


@pytest.mark.parametrize("H,E,I,k,Is,act,T", [
    (256, 32, 128, 8, 256, "f32", 4),      # smallest grouped batch
    (192, 7, 64, 3, 0, "bf16", 37),        # 6 chunks over 4 waves, no shared expert
    (320, 64, 192, 8, 320, "bf16", 53),    # ragged everywhere
    (512, 40, 192, 6, 640, "bf16", 33),    # shared expert wider than the routed ones
    (512, 40, 256, 4, 128, "f32", 20),     # shared expert narrower
    (64, 1, 64, 1, 64, "f32", 40),         # one expert takes all 40 tokens (3 tiles)
    (1024, 1024, 128, 16, 0, "bf16", 70),  # most experts, largest k
    (8192, 16, 64, 2, 128, "bf16", 9),     # largest hidden
    (256, 8, 128, 2, 8192, "bf16", 6),     # wide shared expert (128 groups of I)
])
@pytest.mark.parametrize("bits", [4, 2])
def test_grouped_shapes(orc, H, E, I, k, Is, act, T, bits):
    dl = DeviceLayer(0xB17E0600 + H + E + T, 2, H, E, I, k, Is, act, bits=bits)
    xq, xd = tokens(dl, orc, T)
    ids, w, y = dl.layer_obj.forward(to_dev(xq, act))
    check(dl, orc, xd, ids, w, y, f"{bits}-bit H{H} E{E} I{I} k{k} S{Is} {act} T{T}")


def test_repeated_tokens_fill_many_tiles(orc):
    """One token repeated 45 times among others: each of its experts gets at
    least 45 rows (several 16-row tiles); every copy gives the same result."""
    dl = DeviceLayer(0xB17E0610, 0, 256, 24, 128, 4, 192, "bf16")
    xq, xd = tokens(dl, orc, 6)
    order = [0] * 45 + [1, 2, 3, 4, 5] + [0] * 3
    x = to_dev(xq[order], "bf16")
    ids, w, y = dl.layer_obj.forward(x)
    rows = [i for i, o in enumerate(order) if o == 0]
    for r in rows[1:]:
        assert torch.equal(y[r], y[rows[0]]) and torch.equal(ids[r], ids[rows[0]])
    check(dl, orc, [xd[o] for o in order], ids, w, y, "repeated token", sample=[0, 45, 46, 47, 48, 49])


@pytest.mark.parametrize("bits", [4, 2])
def test_batch_permutation_invariance(orc, bits):
    dl = DeviceLayer(0xB17E0620, 0, 512, 64, 256, 8, 256, "bf16", bits=bits)
    xq, xd = tokens(dl, orc, 48)
    perm = np.random.default_rng(1).permutation(48)
    a = dl.layer_obj.forward(to_dev(xq, "bf16"))
    b = dl.layer_obj.forward(to_dev(xq[perm], "bf16"))
    p = torch.from_numpy(perm).cuda()
    for u, v in zip(a, b):
        assert torch.equal(u[p], v)
    sub = dl.layer_obj.forward(to_dev(xq[10:17], "bf16"))
    for u, v in zip(a, sub):
        assert torch.equal(u[10:17], v)


@pytest.mark.parametrize("bits", [4, 2])
def test_api_expert_outputs_and_fused_forward(orc, bits):
    dl = DeviceLayer(0xB17E0630, 0, 384, 20, 192, 5, 128, "f32", bits=bits)
    xq, xd = tokens(dl, orc, 29)
    x = to_dev(xq, "f32")
    ws = dl.layer_obj.workspace(29)
    ids_f, w_f, y_f = dl.layer_obj.forward(x, ws)
    ids_r, w_r = dl.layer_obj.route(x, ws)
    eo = dl.layer_obj.ffn(x, ids_r, ws)
    y_c = dl.layer_obj.combine(eo, w_r)
    assert torch.equal(ids_f, ids_r) and torch.equal(w_f, w_r) and torch.equal(y_f, y_c)
    eo = eo.cpu().numpy()
    worst = 0.0
    for t in range(29):
        _, _, _, yr, ys = dl.oracle(orc, xd[t])
        for j in range(dl.k):
            worst = max(worst, rel_err(eo[t, j], yr[j]))
        worst = max(worst, rel_err(eo[t, dl.k], ys))
    say(f"{bits}-bit per-slot expert outputs: max rel err {worst:.2e}")
    assert worst <= Y_TOL


def test_no_shared_expert_rows_are_zero(orc):
    dl = DeviceLayer(0xB17E0640, 0, 256, 16, 128, 4, 0, "bf16")
    xq, _ = tokens(dl, orc, 7)
    x = to_dev(xq, "bf16")
    ids, _ = dl.layer_obj.route(x)
    eo = dl.layer_obj.ffn(x, ids)
    assert torch.count_nonzero(eo[:, dl.k]) == 0


def test_bad_ids_raise_device_error_and_poison():
    from bit_routed_expert_moe_amd import MoeError
    dl = DeviceLayer(0xB17E0650, 0, 256, 16, 128, 4, 128, "bf16")
    x = to_dev(synth.quantize_act(synth.activations(1, 0, 0, 256, n_tokens=5), "bf16"), "bf16")
    ws = dl.layer_obj.workspace(5)
    dl.layer_obj.poll_error(ws)
    ids = torch.tensor([[0, 1, 16, 3], [4, -1, 6, 7], [8, 9, 10, 11], [12, 13, 14, 15],
                        [1, 2, 3, 1 << 20]], dtype=torch.int32, device="cuda")
    eo = dl.layer_obj.ffn(x, ids, ws).cpu().numpy()
    with pytest.raises(MoeError) as ei:
        dl.layer_obj.poll_error(ws)
    assert ei.value.status == -8
    dl.layer_obj.poll_error(ws)  # cleared
    bad = {(0, 2), (1, 1), (4, 3)}
    for t in range(5):
        for j in range(5):
            if (t, j) in bad:
                assert np.all(np.isnan(eo[t, j])), (t, j)
            else:
                assert np.all(np.isfinite(eo[t, j])), (t, j)


def test_long_call_runs_in_chunks(orc):
    """A call longer than one grouped pass (here k = 16 and a 16384-wide shared
    expert give 2^31 / (17 * 16384 * 2) = 3855 tokens per pass): tokens on both
    sides of the pass boundary match the oracle and equal a short call on the
    same tokens bit for bit."""
    H, E, I, k, Is, T = 64, 16, 64, 16, 16384, 3900
    per_pass = min(8192, (2 ** 31 - 1) // ((k + 1) * Is * 2), (2 ** 31 - 1) // (H * 2))
    assert per_pass == 3855 < T
    dl = DeviceLayer(0xB17E0660, 0, H, E, I, k, Is, "bf16")
    xq, xd = tokens(dl, orc, T)
    ids, w, y = dl.layer_obj.forward(to_dev(xq, "bf16"))
    lo, hi = per_pass - 5, per_pass + 5
    i2, w2, y2 = dl.layer_obj.forward(to_dev(xq[lo:hi], "bf16"))
    assert torch.equal(i2, ids[lo:hi]) and torch.equal(w2, w[lo:hi]) and torch.equal(y2, y[lo:hi])
    check(dl, orc, xd, ids, w, y, "chunked call", sample=[0, lo, per_pass - 1, per_pass, hi, T - 1])
