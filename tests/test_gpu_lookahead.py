"""Router lookahead (moe_cache_prefetch) through the C ABI (needs a GPU).

A slot-cached layer is given a hint vector before each token and prefetches
the hint's predicted experts:
  * its outputs stay bit-identical to the fully resident layer's;
  * the predicted ids are the oracle's top-k of the hint;
  * hits, misses, prefetch copies issued and prefetched experts later selected
    equal a CPU model of the cache that applies the same placement rules;
  * a hint equal to the token itself makes every selection a hit;
  * bad arguments are rejected on the host.
Hints are noisy previews of the token, rho * x + sqrt(1 - rho^2) * z, the way a
residual stream previews the next layer's input.
"""
import numpy as np
import pytest
import torch

import synth
from _gpu_helpers import DeviceLayer, gap_ok, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


class CacheModel:
    """The slot cache's rules: counts +1 per selection; a miss enters the lowest
    free slot, else replaces the resident expert that is neither pinned nor in
    the protected set with (LFU) the fewest selections, then the oldest use,
    then the lowest slot, or (LRU) the oldest use, then the lowest slot.  A
    prefetch places each predicted expert that is not resident the same way,
    protecting the whole prediction, stamped with the last token's tick, and
    stops when no slot can be taken."""

    def __init__(self, n_slots, n_experts, policy):
        self.n, self.policy = n_slots, policy
        self.holder, self.where = [None] * n_slots, {}
        self.uses, self.stamp = [0] * n_experts, [0] * n_slots
        self.pinned, self.pref = [False] * n_slots, [False] * n_slots
        self.tick = self.hits = self.misses = self.issued = self.used = 0

    def _slot(self, keep):
        free = [q for q, h in enumerate(self.holder) if h is None]
        if free:
            return free[0]
        cands = [q for q in range(self.n)
                 if not self.pinned[q] and self.holder[q] not in keep]
        if not cands:
            return None
        if self.policy == "lru":
            return min(cands, key=lambda q: (self.stamp[q], q))
        return min(cands, key=lambda q: (self.uses[self.holder[q]], self.stamp[q], q))

    def _enter(self, e, q):
        if self.holder[q] is not None:
            del self.where[self.holder[q]]
        self.holder[q], self.where[e] = e, q

    def prefetch(self, pred):
        keep = set(pred)
        for e in pred:
            if e in self.where:
                continue
            q = self._slot(keep)
            if q is None:
                break
            self._enter(e, q)
            self.pref[q], self.stamp[q] = True, self.tick
            self.issued += 1

    def token(self, ids):
        self.tick += 1
        keep = set(ids)
        for e in ids:
            self.uses[e] += 1
            if e in self.where:
                q = self.where[e]
                self.hits += 1
                if self.pref[q]:
                    self.used += 1
                    self.pref[q] = False
            else:
                self.misses += 1
                q = self._slot(keep)
                self._enter(e, q)
                self.pref[q] = False
            self.stamp[q] = self.tick


def cached_twin(dl, n_slots, policy):
    from bit_routed_expert_moe_amd import Layer, record_bytes
    host = torch.empty(dl.pool.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(dl.pool.cpu())
    slots = torch.zeros(n_slots * record_bytes(dl.H, dl.I), dtype=torch.uint8, device="cuda")
    return Layer(dl.H, dl.E, dl.I, dl.k, dl.Is, torch.from_numpy(dl.rq).cuda(),
                 torch.from_numpy(dl.rs.view(np.float16)).cuda(), None, dl.shared, act=dl.act,
                 n_slots=n_slots, host_pool=host, slots=slots, cache_policy=policy), host, slots


def hint_for(orc, dl, xd, step, rho):
    """A seeded noisy preview of xd whose top-(k+1) logits are well separated."""
    for a in range(100):
        z = np.random.default_rng([dl.seed, step, a]).standard_normal(dl.H) * np.std(xd)
        hq = synth.quantize_act(rho * xd + np.sqrt(1.0 - rho * rho) * z, dl.act)
        hd = orc.act_to_f64(dl.act, hq)
        if gap_ok(orc.router_logits(dl.rq, dl.rs, hd), dl.k):
            return hq, hd
    raise RuntimeError("no well-separated hint found")


@pytest.mark.parametrize("policy,n_predict,rho,mode", [
    ("lfu", 8, 0.9, "call"), ("lru", 8, 0.9, "call"), ("lfu", 4, 0.8, "call"),
    ("lru", 3, 0.95, "call"), ("lfu", 8, 0.9, "ids"), ("lru", 5, 0.8, "ids"),
])
def test_prefetch_matches_resident_and_cache_model(orc, policy, n_predict, rho, mode):
    """mode "call": moe_cache_prefetch on the hint; "ids": moe_route_topk on the
    hint, then moe_cache_prefetch_ids with the ids read back on the host."""
    H, E, I, k, Is, n_slots, steps = 512, 48, 192, 8, 256, 12, 32
    dl = DeviceLayer(0xB17E0700 + n_predict, 0, H, E, I, k, Is, "bf16")
    cached, _, _ = cached_twin(dl, n_slots, policy)
    model = CacheModel(n_slots, E, policy)
    ws_r, ws_c = dl.layer_obj.workspace(1), cached.workspace(1)
    recall = 0
    for step in range(steps):
        xq, xd = dl.natural_token(orc, step)
        hq, hd = hint_for(orc, dl, xd, step, rho)
        if mode == "call":
            pred = cached.cache_prefetch(to_dev(hq, "bf16"), n_predict, ws_c)
        else:
            pred = cached.route(to_dev(hq[None], "bf16"), ws_c)[0][0, :n_predict].tolist()
            cached.cache_prefetch_ids(pred)
        want = orc.route(dl.rq, dl.rs, hd, k)[0][:n_predict].tolist()
        assert pred == want, f"step {step}: predicted {pred}, oracle {want}"
        model.prefetch(pred)
        x = to_dev(xq[None], "bf16")
        r = dl.layer_obj.forward(x, ws_r)
        c = cached.forward(x, ws_c)
        for a_, b_ in zip(r, c):
            assert torch.equal(a_, b_), f"step {step}: cached result differs from resident"
        ids = orc.route(dl.rq, dl.rs, xd, k)[0].tolist()
        assert r[0].cpu().numpy()[0].tolist() == ids
        model.token(ids)
        recall += len(set(pred) & set(ids))
    assert cached.cache_stats() == (model.hits, model.misses)
    assert cached.prefetch_stats() == (model.issued, model.used)
    assert model.issued > 0 and model.used > 0
    print(f"{mode} {policy} n_predict={n_predict} rho={rho}: recall {recall / (steps * n_predict):.3f}, "
          f"hits {model.hits} misses {model.misses}, prefetched {model.issued} used {model.used}")


def test_exact_hint_turns_every_selection_into_a_hit(orc):
    dl = DeviceLayer(0xB17E0710, 0, 256, 32, 128, 8, 128, "bf16")
    cached, _, _ = cached_twin(dl, 10, "lfu")
    cached.cache_pin([3, 5])  # 8 unpinned slots: room for a whole prediction
    ws = cached.workspace(1)
    for step in range(12):
        xq, _ = dl.natural_token(orc, step)
        x = to_dev(xq[None], "bf16")
        cached.cache_prefetch(x[0], None, ws)
        ids, w, y = cached.forward(x, ws)
        r = dl.layer_obj.forward(x)
        assert torch.equal(y, r[2]) and torch.equal(ids, r[0])
    hits, misses = cached.cache_stats()
    issued, used = cached.prefetch_stats()
    assert (hits, misses) == (12 * 8, 0)
    assert used == issued > 0


def test_prefetch_argument_errors(orc):
    from bit_routed_expert_moe_amd import MoeError
    dl = DeviceLayer(0xB17E0720, 0, 256, 16, 128, 4, 0, "bf16")
    cached, _, _ = cached_twin(dl, 6, "lfu")
    xq, _ = dl.natural_token(orc, 0)
    x = to_dev(xq, "bf16")
    for n in (0, 5, -1):
        with pytest.raises(MoeError) as ei:
            cached.cache_prefetch(x, n)
        assert ei.value.status == -1, n
    for bad in ([], [0, 1, 2, 3, 4], [1, 1], [16], [-1]):  # n out of 1..k, duplicate, range
        with pytest.raises(MoeError) as ei:
            cached.cache_prefetch_ids(bad)
        assert ei.value.status == -1, bad
    with pytest.raises(MoeError) as ei:
        dl.layer_obj.cache_prefetch(x)  # resident layer: no slot cache
    assert ei.value.status == -7
    with pytest.raises(MoeError) as ei:
        dl.layer_obj.cache_prefetch_ids([0])
    assert ei.value.status == -7
    with pytest.raises(MoeError) as ei:
        dl.layer_obj.prefetch_stats()
    assert ei.value.status == -7


def test_prefetched_slot_evicted_before_use(orc):
    """Wrong predictions of never-selected experts, issued right before a token
    whose selection misses: the LFU evicts exactly those prefetched slots (count
    0), so each miss lands in a slot whose prefetch copy may still be running on
    the side stream.  Such a miss must be copied behind that copy, not beside
    it: the output stays bit-identical to the resident layer's, every step."""
    H, E, I, k, Is, n_slots = 512, 48, 192, 8, 256, 12
    dl = DeviceLayer(0xB17E0730, 0, H, E, I, k, Is, "bf16")
    cached, _, _ = cached_twin(dl, n_slots, "lfu")
    model = CacheModel(n_slots, E, "lfu")
    ws_r, ws_c = dl.layer_obj.workspace(1), cached.workspace(1)
    evicted_prefetch = 0
    for step in range(24):
        xq, xd = dl.natural_token(orc, step)
        ids = orc.route(dl.rq, dl.rs, xd, k)[0].tolist()
        if step >= 2:  # the cache is full: predict experts never selected and not about to be
            pred = [e for e in range(E) if model.uses[e] == 0 and e not in model.where and e not in ids][:k]
            if pred:
                cached.cache_prefetch_ids(pred)
                model.prefetch(pred)
        before = {q: model.holder[q] for q in range(n_slots) if model.pref[q]}
        x = to_dev(xq[None], "bf16")
        r = dl.layer_obj.forward(x, ws_r)
        c = cached.forward(x, ws_c)
        for a_, b_ in zip(r, c):
            assert torch.equal(a_, b_), f"step {step}: cached result differs from resident"
        model.token(ids)
        evicted_prefetch += sum(1 for q, e in before.items() if model.holder[q] != e)
    assert cached.cache_stats() == (model.hits, model.misses)
    assert cached.prefetch_stats() == (model.issued, model.used)
    assert evicted_prefetch >= 8, f"only {evicted_prefetch} prefetched slots were evicted before use"
    print(f"prefetched slots evicted before use: {evicted_prefetch}; misses {model.misses}")
