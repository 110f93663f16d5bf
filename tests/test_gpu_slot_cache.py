"""The HBM expert-slot cache (out-of-core decode) through the C ABI (needs a GPU).

* Outputs are bit-identical to the fully resident layer on the same records.
* Hits and misses equal a CPU simulation of the replacement policy (LFU or
  LRU, with or without a pinned set; written here, independently of the
  library) on the oracle's expert-id stream.
* An unpinned host pool, multi-token calls and bad pin requests are rejected.
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


def cache_simulation(id_stream, n_slots, n_experts, policy="lfu", pin=(), pin_at=0):
    """Counts +1 per selection, never decayed; a miss enters the lowest free slot,
    else replaces a resident expert that is neither pinned nor selected by this
    token: LFU the fewest selections, then least recently used, then lowest
    slot; LRU the least recently used, then lowest slot.  `pin` (applied before
    token `pin_at`) places its experts into free or evicted slots, never to be
    evicted.  Returns (hits, misses, hits on pinned experts after pinning)."""
    where, holder = {}, [None] * n_slots
    uses, stamp, pinned = [0] * n_experts, [0] * n_slots, [False] * n_slots
    hits = misses = pinned_hits = 0
    tick = 0

    def victim(keep):
        cands = [q for q in range(n_slots)
                 if holder[q] is not None and not pinned[q] and holder[q] not in keep]
        if policy == "lru":
            return min(cands, key=lambda q: (stamp[q], q))
        return min(cands, key=lambda q: (uses[holder[q]], stamp[q], q))

    def place(e, keep):
        free = [q for q, h in enumerate(holder) if h is None]
        q = free[0] if free else victim(keep)
        if holder[q] is not None:
            del where[holder[q]]
        holder[q] = e
        where[e] = q
        return q

    for step, ids in enumerate(id_stream):
        if pin and step == pin_at:
            tick += 1
            pinned = [False] * n_slots
            for e in pin:
                q = where[e] if e in where else place(e, set(pin))
                pinned[q] = True
                stamp[q] = tick
        tick += 1
        chosen = set(int(e) for e in ids)
        for e in (int(v) for v in ids):
            uses[e] += 1
            if e in where:
                hits += 1
                q = where[e]
                pinned_hits += int(pinned[q])
            else:
                misses += 1
                q = place(e, chosen)
            stamp[q] = tick
    return hits, misses, pinned_hits


def cached_twin(dl, n_slots, policy="lfu"):
    """A slot-cached layer over the same record bytes as DeviceLayer dl."""
    from bit_routed_expert_moe_amd import Layer, record_bytes
    host = torch.empty(dl.pool.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(dl.pool.cpu())
    slots = torch.zeros(n_slots * record_bytes(dl.H, dl.I), dtype=torch.uint8, device="cuda")
    rq = torch.from_numpy(dl.rq).cuda()
    rs = torch.from_numpy(dl.rs.view(np.float16)).cuda()
    return Layer(dl.H, dl.E, dl.I, dl.k, dl.Is, rq, rs, None, dl.shared, act=dl.act,
                 n_slots=n_slots, host_pool=host, slots=slots, cache_policy=policy), host, slots


@pytest.mark.parametrize("policy,zipf,pin", [
    ("lfu", False, False), ("lfu", True, False), ("lru", True, False),
    ("lfu", True, "stats"), ("lru", True, "stats"), ("lfu", True, "learned"), ("lru", True, "learned"),
])
def test_cached_layer_matches_resident_and_policy(orc, policy, zipf, pin):
    """48 decode steps; with `pin`, the 4 most used experts of the first 16
    steps are pinned before step 16: counted here from the oracle's ids
    ("stats", a statistics pass) or taken by the layer from its own usage
    heatmap ("learned"), which must equal those counts."""
    H, E, I, k, Is, n_slots = 512, 48, 192, 8, 256, 12
    dl = DeviceLayer(0xB17E0500 + zipf, 0, H, E, I, k, Is, "bf16")
    cached, _, _ = cached_twin(dl, n_slots, policy)
    zr = None
    if zipf:
        Wd = dl.rq.astype(np.float64) * dl.rs.view(np.float16).astype(np.float64)[:, None]
        zr = synth.ZipfRealiser(Wd, 1.1, dl.seed, 0)
    ws_r, ws_c = dl.layer_obj.workspace(1), cached.workspace(1)
    oracle_ids, pinned = [], ()
    for step in range(48):
        if pin and step == 16:
            counts = np.bincount(np.concatenate(oracle_ids), minlength=E)
            pinned = tuple(int(e) for e in sorted(range(E), key=lambda e: (-counts[e], e))[:n_slots - k])
            if pin == "stats":
                cached.cache_pin(pinned)
            else:
                assert cached.cache_usage() == counts.tolist()
                cached.cache_pin_hottest(n_slots - k)
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
    sim = cache_simulation(oracle_ids, n_slots, E, policy, pinned, 16)
    assert (hits, misses) == sim[:2]
    assert hits + misses == 48 * k
    if pin:  # every later selection of a pinned expert was a hit
        later = sum(int(e in pinned) for ids in oracle_ids[16:] for e in ids)
        assert sim[2] == later > 0
    print(f"{policy} zipf={zipf} pin={len(pinned)}: hits {hits} misses {misses} "
          f"hit rate {hits / (hits + misses):.3f}")


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
    for bad in ([0, 1, 2, 3, 4], [1, 1], [16], [-1]):  # more than n_slots - k, duplicate, out of range
        with pytest.raises(MoeError) as ei:
            cached.cache_pin(bad)
        assert ei.value.status == -1, bad
    with pytest.raises(MoeError) as ei:
        dl.layer_obj.cache_pin([0])  # no slot cache
    assert ei.value.status == -7


@pytest.mark.timeout(600)
def test_offload_workload_shapes_full_size(orc):
    """The out-of-core workload at its stated shapes: hidden 2816, 256 experts of
    intermediate 704, shared 2112, 16 LFU slots per layer filled from a pinned
    host pool of all 256 records, Zipf(1.1) routing.  Two layers, 512 decode
    steps each (layer 0 then layer 1 per step, one workspace per twin): every
    step's ids, gates and y equal the resident layer's bit for bit, the ids
    equal the oracle's, every 64th step's y is within 2e-3 of the oracle, and
    each layer's hits and misses equal the CPU LFU simulation."""
    from _gpu_helpers import W_TOL, Y_TOL, rel_err, zipf_tokens
    wl = synth.WORKLOADS["offload_h2816_e256_l40_lfu16"]
    NL, S = 2, 512
    dls = [DeviceLayer(wl.seed, l, wl.hidden, wl.n_experts, wl.inter, wl.top_k, wl.shared_inter, wl.act)
           for l in range(NL)]
    twins = [cached_twin(dl, wl.n_slots) for dl in dls]
    toks = [zipf_tokens(dl, orc, wl.zipf_s, range(S)) for dl in dls]
    ws_r, ws_c = dls[0].layer_obj.workspace(1), twins[0][0].workspace(1)
    oracle_ids = [[] for _ in range(NL)]
    worst_y = 0.0
    for step in range(S):
        for l, dl in enumerate(dls):
            xq, xd = toks[l][step]
            x = to_dev(xq[None], wl.act)
            r = dl.layer_obj.forward(x, ws_r)
            c = twins[l][0].forward(x, ws_c)
            for a_, b_ in zip(r, c):
                assert torch.equal(a_, b_), f"layer {l} step {step}: cached result differs from resident"
            if step % 64 == 0:
                rid, rw, ry, _, _ = dl.oracle(orc, xd)
                assert np.max(np.abs(r[1].cpu().numpy()[0] - rw)) <= W_TOL
                worst_y = max(worst_y, rel_err(r[2].cpu().numpy()[0], ry))
            else:
                rid = orc.route(dl.rq, dl.rs, xd, wl.top_k)[0]
            assert r[0].cpu().numpy()[0].tolist() == rid.tolist(), f"layer {l} step {step}"
            oracle_ids[l].append(rid)
    for l in range(NL):
        hits, misses = twins[l][0].cache_stats()
        sim = cache_simulation(oracle_ids[l], wl.n_slots, wl.n_experts, "lfu")
        assert (hits, misses) == sim[:2], f"layer {l}"
        print(f"offload shapes, layer {l}: {S} steps, hits {hits} misses {misses} "
              f"hit rate {hits / (hits + misses):.3f}", flush=True)
    print(f"offload shapes: max rel y err on sampled steps {worst_y:.2e}", flush=True)
    assert worst_y <= Y_TOL


def test_cached_layer_large_hidden_matches_resident(orc):
    """Hidden 4608 (4-wave gate/up units, the shared expert's blocks in slices
    of H): the slot-cached layer launches the shared units and the routed
    units separately, the resident layer in one launch; every step's ids,
    gates and y agree bit for bit, and y is within 2e-3 of the oracle."""
    from _gpu_helpers import Y_TOL, rel_err
    H, E, I, k, Is, n_slots = 4608, 24, 128, 4, 256, 8
    dl = DeviceLayer(0xB17E0530, 0, H, E, I, k, Is, "bf16")
    cached, _, _ = cached_twin(dl, n_slots)
    ws_r, ws_c = dl.layer_obj.workspace(1), cached.workspace(1)
    worst = 0.0
    for step in range(12):
        xq, xd = dl.natural_token(orc, step)
        x = to_dev(xq[None], "bf16")
        r = dl.layer_obj.forward(x, ws_r)
        c = cached.forward(x, ws_c)
        for a_, b_ in zip(r, c):
            assert torch.equal(a_, b_), f"step {step}: cached result differs from resident"
        rid, rw, ry, _, _ = dl.oracle(orc, xd)
        assert r[0].cpu().numpy()[0].tolist() == rid.tolist()
        worst = max(worst, rel_err(r[2].cpu().numpy()[0], ry))
    assert worst <= Y_TOL, worst


def test_saved_heatmap_pins_the_hottest_at_startup(orc, tmp_path):
    """The pages' persistent usage heatmap: the per-expert counts of one run,
    saved to a file, pin the hottest experts of a fresh layer before its first
    token.  Every later selection of a pinned expert is a hit, hits and misses
    equal the simulation with that pinned set, and outputs stay bit-identical
    to the resident layer."""
    H, E, I, k, Is, n_slots = 512, 48, 192, 8, 256, 12
    dl = DeviceLayer(0xB17E0510, 0, H, E, I, k, Is, "bf16")
    Wd = dl.rq.astype(np.float64) * dl.rs.view(np.float16).astype(np.float64)[:, None]
    zr = synth.ZipfRealiser(Wd, 1.1, dl.seed, 0)
    toks = []
    for step in range(40):
        for a in range(50):
            xq = synth.quantize_act(zr.activations(step, a)[0], "bf16")
            xd = orc.act_to_f64("bf16", xq)
            if gap_ok(orc.router_logits(dl.rq, dl.rs, xd), k):
                break
        toks.append((xq, orc.route(dl.rq, dl.rs, xd, k)[0]))
    ws_r = dl.layer_obj.workspace(1)
    first, _, _ = cached_twin(dl, n_slots, "lfu")
    ws_1 = first.workspace(1)
    for xq, _ in toks[:16]:
        first.forward(to_dev(xq[None], "bf16"), ws_1)
    heat = first.cache_usage()
    assert heat == np.bincount(np.concatenate([ids for _, ids in toks[:16]]), minlength=E).tolist()
    np.save(tmp_path / "usage.npy", np.array(heat, dtype=np.uint64))
    saved = np.load(tmp_path / "usage.npy").tolist()
    pinned = tuple(sorted(range(E), key=lambda e: (-saved[e], e))[:n_slots - k])
    second, _, _ = cached_twin(dl, n_slots, "lfu")
    second.cache_pin_hottest(n_slots - k, saved)
    ws_2 = second.workspace(1)
    for step, (xq, ids) in enumerate(toks[16:]):
        x = to_dev(xq[None], "bf16")
        r = dl.layer_obj.forward(x, ws_r)
        c = second.forward(x, ws_2)
        for a_, b_ in zip(r, c):
            assert torch.equal(a_, b_), f"step {16 + step}: cached result differs from resident"
        assert r[0].cpu().numpy()[0].tolist() == ids.tolist()
    sim = cache_simulation([ids for _, ids in toks[16:]], n_slots, E, "lfu", pinned, 0)
    assert second.cache_stats() == sim[:2]
    later = sum(int(e in pinned) for _, ids in toks[16:] for e in ids)
    assert sim[2] == later > 0
    assert second.cache_usage() == np.bincount(np.concatenate([ids for _, ids in toks[16:]]), minlength=E).tolist()
    print(f"saved heatmap pins {pinned}: {later} selections of them, all hits; "
          f"hits {sim[0]} misses {sim[1]}")
