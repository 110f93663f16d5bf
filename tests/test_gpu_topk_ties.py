"""Exact logit ties through the C ABI (needs a GPU).

The router here repeats a few distinct rows (with their fp16 scales) across
all experts, so copies produce exactly equal logits on both sides: the
selection must take every copy of the better rows and then the lowest ids
among the copies at the k-th place, in the order logit descending, lower id
first (the oracle's rule).  Distinct rows are kept more than 1e-4 apart so
that fp32 and fp64 agree on their order.  Covered on the per-token path
(1 and 3 tokens) and on the grouped path (9 tokens), with k = 8 over 40 and
100 experts and k = 16 over 64.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from _gpu_helpers import GAP, W_TOL, Y_TOL, DeviceLayer, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def tied_layer(seed, H, E, I, k, Is, distinct):
    from bit_routed_expert_moe_amd import Layer
    dl = DeviceLayer(seed, 0, H, E, I, k, Is, "bf16")
    base_q, base_s = synth.router(seed, 1, distinct, H)
    dl.rq = np.ascontiguousarray(base_q[np.arange(E) % distinct])
    dl.rs = np.ascontiguousarray(base_s[np.arange(E) % distinct])
    dl.layer_obj = Layer(H, E, I, k, Is, torch.from_numpy(dl.rq).cuda(),
                         torch.from_numpy(dl.rs.view(np.float16)).cuda(), dl.pool, dl.shared, act="bf16")
    return dl


def tied_tokens(dl, orc, n):
    """Tokens whose distinct logit values covering the top k+1 entries are
    separated by more than GAP (copies tie exactly)."""
    out = []
    for step in range(10 * n + 50):
        x = synth.activations(dl.seed, 7, step, dl.H)[0]
        xq = synth.quantize_act(x, "bf16")
        xd = orc.act_to_f64("bf16", xq)
        lg = orc.router_logits(dl.rq, dl.rs, xd)
        u = np.unique(lg)[::-1]
        counts = [(lg == v).sum() for v in u]
        need = np.searchsorted(np.cumsum(counts), dl.k + 1) + 1
        if np.all(-np.diff(u[:need + 1]) > GAP):
            out.append((xq, xd))
            if len(out) == n:
                return out
    raise RuntimeError("no separated token found")


@pytest.mark.parametrize("E,k,distinct,T", [
    (40, 8, 8, 1), (40, 8, 8, 3), (40, 8, 8, 9),
    (100, 8, 8, 1), (100, 8, 8, 9),
    (64, 16, 16, 2), (64, 16, 16, 9),
])
def test_exact_ties_break_to_lower_id(orc, E, k, distinct, T):
    H, I, Is = 256, 128, 128
    dl = tied_layer(0xB17E0700 + E + k, H, E, I, k, Is, distinct)
    toks = tied_tokens(dl, orc, T)
    x = to_dev(np.stack([t[0] for t in toks]), "bf16")
    ids, w, y = dl.layer_obj.forward(x)
    ids_r, w_r = dl.layer_obj.route(x)
    assert torch.equal(ids, ids_r) and torch.equal(w, w_r)
    ids, w, y = ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()
    worst_w = worst_y = 0.0
    n_tied = 0
    for t, (_, xd) in enumerate(toks):
        rid, rw, ry, _, _ = dl.oracle(orc, xd)
        lg = orc.router_logits(dl.rq, dl.rs, xd)
        n_tied += int(np.sum(lg == lg[rid[-1]]) > 1)  # a tie at the k-th place
        assert ids[t].tolist() == rid.tolist(), f"token {t}: {ids[t]} vs {rid}"
        worst_w = max(worst_w, float(np.max(np.abs(w[t] - rw))))
        worst_y = max(worst_y, rel_err(y[t], ry))
    print(f"E{E} k{k} T{T}: {n_tied}/{T} tokens tied at the k-th place; "
          f"max |w err| {worst_w:.2e}, max rel y err {worst_y:.2e}", flush=True)
    assert n_tied == T  # every token exercises the tie rule at the boundary
    assert worst_w <= W_TOL and worst_y <= Y_TOL
