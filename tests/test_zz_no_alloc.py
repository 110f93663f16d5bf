"""moe_layer_forward_noalloc (the workspace in the library's static device
array) against moe_layer_forward with a caller's workspace, through the C ABI
(needs a GPU): ids, gates and outputs bit-identical, on two calls in a row
with the second smaller, on three layers of different shapes; a call whose
workspace would exceed the array is refused before any launch."""
import numpy as np
import pytest
import torch

from _gpu_helpers import DeviceLayer, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _outs(T, k, H):
    return (torch.full((T, k), -7, dtype=torch.int32, device="cuda"),
            torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda"),
            torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda"))


def test_noalloc_forward_matches_workspace_forward(orc):
    big = DeviceLayer(0xA110C001, 0, 2816, 128, 704, 8, 2112, "bf16")   # Gemma-scale shapes
    small = DeviceLayer(0xA110C002, 0, 512, 40, 192, 6, 320, "f32")
    # above hidden 4096: the router launch, and the shared expert in quarters of H
    wide = DeviceLayer(0xA110C004, 0, 6144, 64, 512, 8, 512, "bf16")
    for dl, T1, T2 in ((big, 3, 1), (small, 2, 1), (wide, 3, 2), (big, 1, 1)):
        toks = [dl.natural_token(orc, s) for s in range(T1)]
        xq = np.stack([t[0] for t in toks])
        for T in (T1, T2):  # two calls in a row, the second not larger
            x = to_dev(xq[:T], dl.act)
            ref = dl.layer_obj.forward(x, dl.layer_obj.workspace(T))
            got = dl.layer_obj.forward_noalloc(x, _outs(T, dl.k, dl.H))
            for a_, b_ in zip(ref, got):
                assert torch.equal(a_, b_), f"H{dl.H} T={T}"
            rid = dl.oracle(orc, toks[0][1])[0]
            assert got[0][0].cpu().numpy().tolist() == rid.tolist()


def test_noalloc_refuses_calls_beyond_its_scratch():
    from bit_routed_expert_moe_amd import MoeError
    dl = DeviceLayer(0xA110C003, 0, 2816, 128, 704, 8, 2112, "bf16")
    T = 512  # a grouped call whose workspace is far above 8 MiB
    assert dl.layer_obj.workspace_bytes(T) > (8 << 20)
    x = torch.zeros(T, 2816, dtype=torch.bfloat16, device="cuda")
    outs = _outs(T, 8, 2816)
    with pytest.raises(MoeError) as ei:
        dl.layer_obj.forward_noalloc(x, outs)
    assert ei.value.status == -2
    assert torch.all(outs[0] == -7)  # nothing was launched
