"""Workspace reuse on the per-token (decode) path through the C ABI (needs a GPU).

The down kernel's arrival counters live at fixed offsets at the start of the
workspace and every call returns them to zero, so many calls back to back on
one workspace, calls of other sizes on the same workspace, and replays of a
captured graph all give the same bits as a fresh workspace.
"""
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


def test_back_to_back_and_across_sizes(orc):
    dl = DeviceLayer(0xB17E0710, 0, 512, 64, 256, 8, 256, "bf16")
    toks = [dl.natural_token(orc, s)[0] for s in range(40)]
    ref = [dl.layer_obj.forward(to_dev(t[None], "bf16")) for t in toks]  # fresh workspace each
    ws = dl.layer_obj.workspace(32)
    outs = [dl.layer_obj.forward(to_dev(t[None], "bf16"), ws) for t in toks]  # no sync between
    torch.cuda.synchronize()
    for r, o in zip(ref, outs):
        for a, b in zip(r, o):
            assert torch.equal(a, b)
    # the same workspace for a 32-token call, a 2-token call, then single tokens again
    dl.layer_obj.forward(to_dev(np.stack(toks[:32]), "bf16"), ws)
    two = dl.layer_obj.forward(to_dev(np.stack(toks[:2]), "bf16"), ws)
    for i in (0, 1):
        assert torch.equal(two[2][i], ref[i][2][0])
    for i in (5, 17, 33):
        for a, b in zip(ref[i], dl.layer_obj.forward(to_dev(toks[i][None], "bf16"), ws)):
            assert torch.equal(a, b)
    dl.layer_obj.poll_error(ws)


def test_graph_replays_match_eager(orc):
    dl = DeviceLayer(0xB17E0720, 0, 1024, 64, 256, 8, 512, "bf16")
    toks = [dl.natural_token(orc, s)[0] for s in range(4)]
    xs = [to_dev(t[None], "bf16") for t in toks]
    ws = dl.layer_obj.workspace(1)
    eager = [dl.layer_obj.forward(x, ws) for x in xs]
    outs = [(torch.empty(1, 8, dtype=torch.int32, device="cuda"),
             torch.empty(1, 8, dtype=torch.float32, device="cuda"),
             torch.empty(1, 1024, dtype=torch.float32, device="cuda")) for _ in xs]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x, o in zip(xs, outs):
            dl.layer_obj.forward(x, ws, out=o)
    for rep in range(3):
        for o in outs:
            for t in o:
                t.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for e, o in zip(eager, outs):
            for a, b in zip(e, o):
                assert torch.equal(a, b), f"replay {rep} differs from the eager result"
        dl.layer_obj.forward(xs[0], ws)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
    dl.layer_obj.poll_error(ws)
