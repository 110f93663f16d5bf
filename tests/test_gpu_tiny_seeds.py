"""The tiny single-layer workload (hidden 256, 32 experts of intermediate 128,
top-8, shared expert 256, fp32 activations, one token) over 1,000 seeds: each
seed draws its own router, records and activations, and the one token goes
through the per-token path (a call of one token) and is checked against the
oracle: ids bit-exact, gates within 1e-6, y within 2e-3."""
import numpy as np
import pytest
import torch

import synth
from _gpu_helpers import W_TOL, Y_TOL, DeviceLayer, elem_err, rel_err, to_dev

pytestmark = pytest.mark.gpu

N_SEEDS = 1000


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def test_tiny_layer_one_token_over_many_seeds(orc):
    wl = synth.WORKLOADS["tiny_h256_e32"]
    worst_y = worst_w = worst_e = 0.0
    ws = None
    for i in range(N_SEEDS):
        seed = wl.seed + (i << 16)
        dl = DeviceLayer(seed, 0, wl.hidden, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter, wl.act)
        if ws is None:
            ws = dl.layer_obj.workspace(1)
        xq, xd = dl.natural_token(orc, 0)
        ids, w, y = dl.layer_obj.forward(to_dev(xq[None], wl.act), ws)
        rid, rw, ry, _, _ = dl.oracle(orc, xd)
        assert ids.cpu().numpy()[0].tolist() == rid.tolist(), f"seed {seed:#x}"
        worst_w = max(worst_w, float(np.max(np.abs(w.cpu().numpy()[0] - rw))))
        yh = y.cpu().numpy()[0]
        worst_y = max(worst_y, rel_err(yh, ry))
        worst_e = max(worst_e, elem_err(yh, ry))
        assert worst_w <= W_TOL and worst_y <= Y_TOL, f"seed {seed:#x}"
    print(f"tiny layer over {N_SEEDS} seeds (T=1): max |w err| {worst_w:.2e}, max rel y err "
          f"{worst_y:.2e}, element-wise (floor 1e-3 max|y|) {worst_e:.2e}", flush=True)
