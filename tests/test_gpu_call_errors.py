"""Argument errors of the compute calls, on a real layer handle (needs a GPU).

Token counts outside 1 .. 2^20, misaligned activations or workspace and null
outputs are rejected on the host with the documented status before any launch;
a call that follows them on the same workspace still gives the oracle's
selection and the same bits as a fresh workspace (a rejected call leaves the
workspace's counters and logit words untouched).
"""
import numpy as np
import pytest
import torch

from _gpu_helpers import DeviceLayer, to_dev

pytestmark = pytest.mark.gpu

ARG, ALIGN = -1, -3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def test_compute_calls_reject_bad_arguments(orc):
    from bit_routed_expert_moe_amd import layer as L
    lib = L.lib()
    dl = DeviceLayer(0xE1105000, 0, 512, 48, 192, 8, 256, "bf16")
    h = dl.layer_obj.handle
    xq, xd = dl.natural_token(orc, 0)
    x = to_dev(np.stack([xq, xq]), "bf16")
    ws = dl.layer_obj.workspace(2)
    ids = torch.empty(2, 8, dtype=torch.int32, device="cuda")
    w = torch.empty(2, 8, dtype=torch.float32, device="cuda")
    y = torch.empty(2, 512, dtype=torch.float32, device="cuda")
    eo = torch.empty(2, 9, 512, dtype=torch.float32, device="cuda")
    p = lambda t: t.data_ptr()

    for T in (0, -1, (1 << 20) + 1):
        assert lib.moe_layer_forward(h, p(x), T, p(ids), p(w), p(y), p(ws), None) == ARG, T
        assert lib.moe_route_topk(h, p(x), T, p(ids), p(w), p(ws), None) == ARG, T
        assert lib.moe_expert_ffn(h, p(x), T, p(ids), p(ws), p(eo), None) == ARG, T
    assert lib.moe_layer_forward(h, p(x) + 2, 1, p(ids), p(w), p(y), p(ws), None) == ALIGN
    assert lib.moe_layer_forward(h, p(x), 1, p(ids), p(w), p(y), p(ws) + 128, None) == ALIGN
    assert lib.moe_layer_forward(h, p(x), 1, None, p(w), p(y), p(ws), None) == ARG
    assert lib.moe_layer_forward(h, p(x), 1, p(ids), p(w), None, p(ws), None) == ARG
    assert lib.moe_layer_forward(h, None, 1, p(ids), p(w), p(y), p(ws), None) == ARG
    assert lib.moe_layer_forward(h, p(x), 1, p(ids), p(w), p(y), None, None) == ARG
    assert lib.moe_route_topk(h, p(x), 1, None, p(w), p(ws), None) == ARG
    assert lib.moe_expert_ffn(h, p(x), 1, None, p(ws), p(eo), None) == ARG
    assert lib.moe_last_error()  # the message of the last rejection

    got = dl.layer_obj.forward(x, ws)
    fresh = dl.layer_obj.forward(x, dl.layer_obj.workspace(2))
    for a_, b_ in zip(got, fresh):
        assert torch.equal(a_, b_)
    want = dl.oracle(orc, xd)[0].tolist()
    assert got[0].cpu().numpy().tolist() == [want, want]
