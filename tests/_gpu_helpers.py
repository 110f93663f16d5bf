"""Shared pieces of the GPU tests: building layers on the device from the seeded
generator, and oracle references computed from the generator's CPU output only
(nothing the GPU path produced is fed to the oracle)."""
from __future__ import annotations

import numpy as np
import torch

import synth
import synth.gpu

Y_TOL = 2e-3   # max |y - y_ref| / max |y_ref| per token
W_TOL = 1e-6   # max |w - w_ref|
GAP = 1e-4     # required separation of the top-(k+1) oracle logits
GAP_SIGMOID = 1e-5  # the same for the sigmoid router's selection keys (score + bias)


def rel_err(y, y_ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    return float(np.max(np.abs(y - y_ref)) / max(np.max(np.abs(y_ref)), 1e-30))


def elem_err(y, y_ref, floor: float = 1e-3) -> float:
    """Element-wise relative error with a floor: max_i |y_i - y_ref_i| /
    max(|y_ref_i|, floor * max |y_ref|) (reported beside rel_err; near-zero
    outputs would otherwise dominate)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.maximum(np.abs(y_ref), floor * max(np.max(np.abs(y_ref)), 1e-30))
    return float(np.max(np.abs(y - y_ref) / den))


def gap_ok(logits: np.ndarray, k: int, gap: float = GAP) -> bool:
    s = np.sort(logits)[::-1][:k + 1]
    return bool(np.all(-np.diff(s) > gap))


class DeviceLayer:
    """One layer's weights on the GPU (router from numpy, records from the GPU
    fill) plus the host copies the oracle needs (router only; records are
    regenerated on the CPU on demand)."""

    def __init__(self, seed, layer, H, E, I, k, Is, act, dev="cuda", gate="softmax",
                 routed_scale=1.0, bias=None, bits=4):
        """gate / routed_scale / bias (float32 numpy [E] or None): the router's
        gate function, as in bit_routed_expert_moe_amd.Layer; bits: code width
        of the expert records (4 or 2)."""
        from bit_routed_expert_moe_amd import Layer, record_bytes
        self.seed, self.layer, self.H, self.E, self.I, self.k, self.Is, self.act = \
            seed, layer, H, E, I, k, Is, act
        self.gate, self.routed_scale, self.bits = gate, routed_scale, bits
        self.bias = None if bias is None else np.asarray(bias, dtype=np.float32)
        self.bias_dev = None if bias is None else torch.from_numpy(self.bias).to(dev)
        self.rq, self.rs = synth.router(seed, layer, E, H)
        self.pool = torch.empty(E * record_bytes(H, I, bits), dtype=torch.uint8, device=dev)
        synth.gpu.fill_records(self.pool, H, I, seed, layer, 0, E, bits=bits)
        self.shared = None
        if Is:
            self.shared = torch.empty(record_bytes(H, Is, bits), dtype=torch.uint8, device=dev)
            synth.gpu.fill_records(self.shared, H, Is, seed, layer, -1, 1, bits=bits)
        self.layer_obj = Layer(H, E, I, k, Is, torch.from_numpy(self.rq).to(dev),
                               torch.from_numpy(self.rs.view(np.float16)).to(dev), self.pool,
                               self.shared, act=act, gate=gate, routed_scale=routed_scale,
                               selection_bias=self.bias_dev, bits=bits)
        self._rec_cache = {}

    def record(self, e: int) -> np.ndarray:
        if e not in self._rec_cache:
            if e == synth.SHARED_INDEX:
                self._rec_cache[e] = synth.expert_record(self.seed, self.layer, e, self.H, self.Is,
                                                         bits=self.bits)
            else:
                self._rec_cache[e] = synth.expert_record(self.seed, self.layer, e, self.H, self.I,
                                                         bits=self.bits)
        return self._rec_cache[e]

    def natural_token(self, orc, step: int, max_attempts: int = 200):
        """Seeded N(0,1) activations for (layer, step), redrawn until the oracle's
        top-(k+1) logits are separated by more than GAP.  Returns (raw, float64)."""
        for a in range(max_attempts):
            x = synth.activations(self.seed, self.layer, step, self.H, attempt=a)[0]
            xq = synth.quantize_act(x, self.act)
            xd = orc.act_to_f64(self.act, xq)
            if gap_ok(self.selection_keys(orc, xd), self.k, GAP if self.gate == "softmax" else GAP_SIGMOID):
                return xq, xd
        raise RuntimeError("no well-separated token found")

    def selection_keys(self, orc, xd: np.ndarray) -> np.ndarray:
        """The oracle's selection keys: logits, or logistic scores plus bias."""
        lg = orc.router_logits(self.rq, self.rs, xd)
        if self.gate == "softmax":
            return lg
        key = 1.0 / (1.0 + np.exp(-lg))
        return key if self.bias is None else key + self.bias.astype(np.float64)

    def oracle(self, orc, xd: np.ndarray):
        ids, w, lg = orc.route(self.rq, self.rs, xd, self.k, gate=self.gate,
                               bias=None if self.bias is None else self.bias.astype(np.float64),
                               scale=self.routed_scale)
        yr = np.stack([orc.expert_ffn(self.H, self.I, self.record(int(e)), xd, bits=self.bits)
                       for e in ids])
        ys = (orc.expert_ffn(self.H, self.Is, self.record(synth.SHARED_INDEX), xd, bits=self.bits)
              if self.Is else None)
        return ids, w, orc.combine(w, yr, ys), yr, ys


def zipf_tokens(dl, orc, zipf_s: float, steps, max_attempts: int = 50):
    """Activations for dl's layer whose router response aims at Zipf(zipf_s)
    Gumbel-top-k targets (synth.ZipfRealiser), one per step, redrawn until the
    oracle's top-(k+1) logits are separated by more than GAP.  [(raw, float64)]."""
    Wd = dl.rq.astype(np.float64) * dl.rs.view(np.float16).astype(np.float64)[:, None]
    zr = synth.ZipfRealiser(Wd, zipf_s, dl.seed, dl.layer)
    out = []
    for step in steps:
        for a in range(max_attempts):
            xq = synth.quantize_act(zr.activations(step, a)[0], dl.act)
            xd = orc.act_to_f64(dl.act, xq)
            if gap_ok(orc.router_logits(dl.rq, dl.rs, xd), dl.k):
                break
        else:
            raise RuntimeError("no well-separated token found")
        out.append((xq, xd))
    return out


def to_dev(xq: np.ndarray, act: str, dev="cuda") -> torch.Tensor:
    if act == "bf16":
        return torch.from_numpy(np.ascontiguousarray(xq).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(xq, dtype=np.float32)).to(dev)
