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

ARG, SHAPE, ALIGN = -1, -2, -3


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


def test_stack_rejects_layers_that_would_overlap():
    """moe_stack_forward places layer l's ids/w at l*T*top_k and its x at
    l*x_stride elements of one dtype: layers of different top_k or activation
    dtype, and strides shorter than a layer's [T][H] block, are refused on the
    host (MOE_ERR_SHAPE) before anything is enqueued; the binding refuses
    them too."""
    import ctypes as C
    from bit_routed_expert_moe_amd import layer as L, stack_forward
    lib = L.lib()
    a = DeviceLayer(0xE1105100, 0, 256, 16, 128, 8, 0, "bf16")
    b = DeviceLayer(0xE1105101, 1, 256, 16, 128, 4, 0, "bf16")  # another top_k
    c = DeviceLayer(0xE1105102, 2, 256, 16, 128, 8, 0, "f32")   # another activation dtype
    ws = a.layer_obj.workspace(1)
    x = torch.zeros(2, 1, 256, dtype=torch.bfloat16, device="cuda")
    ids = torch.full((2, 1, 8), -5, dtype=torch.int32, device="cuda")
    w = torch.zeros(2, 1, 8, dtype=torch.float32, device="cuda")
    y = torch.zeros(2, 1, 256, dtype=torch.float32, device="cuda")
    p = lambda t: t.data_ptr()

    def stack(l0, l1, xs=256, ys=256):
        arr = (C.c_void_p * 2)(l0.layer_obj.handle.value, l1.layer_obj.handle.value)
        return lib.moe_stack_forward(arr, 2, p(x), xs, 1, p(ids), p(w), p(y), ys, p(ws), None)

    assert stack(a, b) == SHAPE and stack(a, c) == SHAPE
    assert stack(a, a, xs=128) == SHAPE and stack(a, a, ys=255) == SHAPE
    torch.cuda.synchronize()
    assert torch.all(ids == -5)  # nothing ran
    assert stack(a, a) == 0      # the same stack with full strides runs
    with pytest.raises(ValueError):
        stack_forward([a.layer_obj, b.layer_obj], x, ws)
