"""The HBM expert-slot cache (out-of-core decode) through the C ABI (needs a GPU).

* Outputs are bit-identical to the fully resident layer on the same records.
* Hits and misses equal a CPU simulation of the LFU policy (written here,
  independently of the library) on the oracle's expert-id stream.
* An unpinned host pool and multi-token calls are rejected.
"""
import numpy as np
import pytest
import torch

import synth
import synth.gpu
from _gpu_helpers import DeviceLayer, gap_ok, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def lfu_simulation(id_stream, n_slots, n_experts):
    """Counts +1 per selection, never decayed; a miss enters the lowest free slot,
    else replaces the resident expert not selected by this token with the fewest
    selections, then least recently used, then lowest slot."""
    where = {}                      # expert -> slot
    holder = [None] * n_slots       # slot -> expert
    uses = [0] * n_experts
    stamp = [0] * n_slots
    hits = misses = 0
    for step, ids in enumerate(id_stream, start=1):
        chosen = set(int(e) for e in ids)
        for e in (int(v) for v in ids):
            uses[e] += 1
            if e in where:
                hits += 1
                s = where[e]
            else:
                misses += 1
                free = [q for q, h in enumerate(holder) if h is None]
                if free:
                    s = free[0]
                else:
                    s = min((q for q in range(n_slots) if holder[q] not in chosen),
                            key=lambda q: (uses[holder[q]], stamp[q], q))
                    del where[holder[s]]
                holder[s] = e
                where[e] = s
            stamp[s] = step
    return hits, misses


def cached_twin(dl, n_slots):
    """A slot-cached layer over the same record bytes as DeviceLayer dl."""
    from bit_routed_expert_moe_amd import Layer, record_bytes
    host = torch.empty(dl.pool.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(dl.pool.cpu())
    slots = torch.zeros(n_slots * record_bytes(dl.H, dl.I), dtype=torch.uint8, device="cuda")
    rq = torch.from_numpy(dl.rq).cuda()
    rs = torch.from_numpy(dl.rs.view(np.float16)).cuda()
    return Layer(dl.H, dl.E, dl.I, dl.k, dl.Is, rq, rs, None, dl.shared, act=dl.act,
                 n_slots=n_slots, host_pool=host, slots=slots), host, slots


@pytest.mark.parametrize("zipf", [False, True])
def test_cached_layer_matches_resident_and_lfu(orc, zipf):
    H, E, I, k, Is, n_slots = 512, 48, 192, 8, 256, 12
    dl = DeviceLayer(0xB17E0500 + zipf, 0, H, E, I, k, Is, "bf16")
    cached, _, _ = cached_twin(dl, n_slots)
    zr = None
    if zipf:
        Wd = dl.rq.astype(np.float64) * dl.rs.view(np.float16).astype(np.float64)[:, None]
        zr = synth.ZipfRealiser(Wd, 1.1, dl.seed, 0)
    ws_r, ws_c = dl.layer_obj.workspace(1), cached.workspace(1)
    oracle_ids = []
    for step in range(48):
        if zr is None:
            xq, xd = dl.natural_token(orc, step)
        else:
            for a in range(50):
                xq = synth.quantize_act(zr.activations(step, a)[0], "bf16")
                xd = orc.act_to_f64("bf16", xq)
                if gap_ok(orc.router_logits(dl.rq, dl.rs, xd), k):
                    break
        oracle_ids.append(orc.route(dl.rq, dl.rs, xd, k)[0])
        x = to_dev(xq[None], "bf16")
        r = dl.layer_obj.forward(x, ws_r)
        c = cached.forward(x, ws_c)
        for a_, b_ in zip(r, c):
            assert torch.equal(a_, b_), f"step {step}: cached result differs from resident"
        assert r[0].cpu().numpy()[0].tolist() == oracle_ids[-1].tolist()
    hits, misses = cached.cache_stats()
    assert (hits, misses) == lfu_simulation(oracle_ids, n_slots, E)
    assert hits + misses == 48 * k
    print(f"zipf={zipf}: hits {hits} misses {misses} hit rate {hits / (hits + misses):.3f}")


def test_cached_api_expert_outputs_match_resident(orc):
    dl = DeviceLayer(0xB17E0510, 0, 256, 32, 128, 4, 128, "bf16")
    cached, _, _ = cached_twin(dl, 6)
    for step in range(12):
        xq, _ = dl.natural_token(orc, step)
        x = to_dev(xq[None], "bf16")
        ids, w = dl.layer_obj.route(x)
        eo_r = dl.layer_obj.ffn(x, ids)
        eo_c = cached.ffn(x, ids)
        assert torch.equal(eo_r, eo_c)


def test_cache_rejects_unpinned_pool_and_batches():
    from bit_routed_expert_moe_amd import Layer, MoeError, record_bytes
    dl = DeviceLayer(0xB17E0520, 0, 256, 16, 128, 4, 0, "bf16")
    rq = torch.from_numpy(dl.rq).cuda()
    rs = torch.from_numpy(dl.rs.view(np.float16)).cuda()
    slots = torch.zeros(8 * record_bytes(256, 128), dtype=torch.uint8, device="cuda")
    plain = torch.empty(dl.pool.numel(), dtype=torch.uint8)  # pageable
    import bit_routed_expert_moe_amd.layer as BL
    import ctypes as C
    d = BL.Desc(256, 16, 128, 4, 0, 64, 1, 0, 8)
    w = BL.Weights(rq.data_ptr(), rs.data_ptr(), None, None, plain.data_ptr(), slots.data_ptr())
    h = C.c_void_p()
    assert BL.lib().moe_layer_create(C.byref(d), C.byref(w), C.byref(h)) == -6
    cached, _, _ = cached_twin(dl, 8)
    x = to_dev(synth.quantize_act(synth.activations(3, 0, 0, 256, n_tokens=2), "bf16"), "bf16")
    with pytest.raises(MoeError) as ei:
        cached.forward(x)
    assert ei.value.status == -7
