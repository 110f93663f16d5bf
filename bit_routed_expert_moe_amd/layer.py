"""ctypes binding of libmoe_layer.so: argument marshalling for torch tensors.

Every compute call goes to the HIP library on the caller's current torch
stream.  The library must have been built (``__graft_entry__.build()``); if it
is missing, loading fails with an error instead of falling back to anything.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LAYER_LIB names another build of the same library (the sanitizer tests
# load one with instrumented host code); by default the in-tree build is loaded
LIB_PATH = os.environ.get("MOE_LAYER_LIB") or os.path.join(HERE, "libmoe_layer.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX_TOPK = 0
MOE_SIGMOID_TOPK = 1
MOE_CACHE_LFU, MOE_CACHE_LRU = 0, 1
STATUS = {0: "MOE_OK", -1: "MOE_ERR_ARG", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_ALIGN",
          -4: "MOE_ERR_HIP", -5: "MOE_ERR_NOMEM", -6: "MOE_ERR_NOT_PINNED",
          -7: "MOE_ERR_STATE", -8: "MOE_ERR_DEVICE"}

EXPORTS = ["moe_expert_record_bytes", "moe_expert_record_bytes_bits", "moe_layer_create", "moe_layer_destroy",
           "moe_workspace_bytes", "moe_route_topk", "moe_expert_ffn", "moe_combine",
           "moe_layer_forward", "moe_layer_forward_noalloc", "moe_stack_forward", "moe_cache_stats", "moe_cache_pin",
           "moe_cache_usage", "moe_cache_pin_hottest",
           "moe_cache_prefetch", "moe_cache_prefetch_ids", "moe_cache_prefetch_stats",
           "moe_poll_device_error", "moe_stream_read",
           "moe_profile_start", "moe_profile_stop", "moe_profile_read",
           "moe_status_str", "moe_last_error"]
KERNEL_NAMES = {0: "route", 1: "prep", 2: "gate_up", 3: "down_combine", 4: "combine", 5: "topk",
                6: "grouped_prep", 7: "grouping", 8: "grouped_gate_up", 9: "grouped_down",
                10: "stream_read"}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Desc(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_experts", C.c_int32), ("inter", C.c_int32),
                ("top_k", C.c_int32), ("shared_inter", C.c_int32), ("group", C.c_int32),
                ("act_dtype", C.c_int32), ("gate_fn", C.c_int32), ("n_slots", C.c_int32),
                ("routed_scale", C.c_float), ("cache_policy", C.c_int32), ("bits", C.c_int32),
                ("reserved", C.c_int32 * 4)]


class Weights(C.Structure):
    _fields_ = [("router_q", C.c_void_p), ("router_scale", C.c_void_p),
                ("experts", C.c_void_p), ("shared", C.c_void_p),
                ("host_pool", C.c_void_p), ("slots", C.c_void_p), ("selection_bias", C.c_void_p)]


_LIB: C.CDLL | None = None


def lib() -> C.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        L.moe_expert_record_bytes.argtypes = [i32, i32]
        L.moe_expert_record_bytes.restype = C.c_size_t
        L.moe_expert_record_bytes_bits.argtypes = [i32, i32, i32]
        L.moe_expert_record_bytes_bits.restype = C.c_size_t
        L.moe_layer_create.argtypes = [C.POINTER(Desc), C.POINTER(Weights), C.POINTER(vp)]
        L.moe_layer_destroy.argtypes = [vp]
        L.moe_workspace_bytes.argtypes = [vp, i32]
        L.moe_workspace_bytes.restype = C.c_size_t
        L.moe_route_topk.argtypes = [vp, vp, i32, vp, vp, vp, vp]
        L.moe_expert_ffn.argtypes = [vp, vp, i32, vp, vp, vp, vp]
        L.moe_combine.argtypes = [vp, vp, vp, i32, vp, i32, vp]
        L.moe_layer_forward.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp]
        L.moe_layer_forward_noalloc.argtypes = [vp, vp, i32, vp, vp, vp, vp]
        L.moe_stack_forward.argtypes = [vp, i32, vp, i64, i32, vp, vp, vp, i64, vp, vp]
        L.moe_poll_device_error.argtypes = [vp, vp, vp]
        L.moe_stream_read.argtypes = [vp, C.c_size_t, i32, vp, vp]
        L.moe_cache_stats.argtypes = [vp, C.POINTER(C.c_uint64), C.POINTER(C.c_uint64)]
        L.moe_cache_pin.argtypes = [vp, C.POINTER(C.c_int32), i32, vp]
        L.moe_cache_usage.argtypes = [vp, C.POINTER(C.c_uint64)]
        L.moe_cache_pin_hottest.argtypes = [vp, C.POINTER(C.c_uint64), i32, vp]
        L.moe_cache_prefetch.argtypes = [vp, vp, i32, vp, C.POINTER(C.c_int32), vp]
        L.moe_cache_prefetch_ids.argtypes = [vp, C.POINTER(C.c_int32), i32, vp]
        L.moe_cache_prefetch_stats.argtypes = [vp, C.POINTER(C.c_uint64), C.POINTER(C.c_uint64)]
        L.moe_status_str.argtypes = [i32]
        L.moe_status_str.restype = C.c_char_p
        L.moe_last_error.restype = C.c_char_p
        L.moe_profile_start.argtypes = [i32]
        L.moe_profile_read.argtypes = [vp, vp, i32]
        L.moe_profile_read.restype = i32
        for f in ["moe_layer_create", "moe_layer_destroy", "moe_route_topk", "moe_expert_ffn",
                  "moe_combine", "moe_layer_forward", "moe_layer_forward_noalloc", "moe_stack_forward",
                  "moe_poll_device_error", "moe_stream_read", "moe_profile_start", "moe_profile_stop",
                  "moe_cache_stats", "moe_cache_pin", "moe_cache_usage", "moe_cache_pin_hottest",
                  "moe_cache_prefetch", "moe_cache_prefetch_ids",
                  "moe_cache_prefetch_stats"]:
            getattr(L, f).restype = i32
        _LIB = L
    return _LIB


def _check(status: int):
    if status != 0:
        raise MoeError(status, lib().moe_last_error().decode())


def record_bytes(hidden: int, inter: int, bits: int = 4) -> int:
    return int(lib().moe_expert_record_bytes_bits(hidden, inter, bits))


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


class Layer:
    """One MoE layer over caller-owned device tensors.

    router_q      int8 [E][H]
    router_scale  float16 [E] (or int16 holding fp16 bits)
    experts       uint8 [E * record_bytes(H, inter, bits)]
    shared        uint8 [record_bytes(H, shared_inter, bits)] or None
    act           "bf16" or "f32" activations
    n_slots       > 0: HBM slot cache of that many records, filled from
    host_pool     pinned uint8 CPU tensor of all E records, into
    slots         uint8 CUDA tensor [n_slots * record_bytes(H, inter)]
                  (experts may then be None)
    gate          "softmax" (renormalised softmax over the selected logits) or
                  "sigmoid" (logistic scores, selection by score + selection_bias,
                  gates = routed_scale * score / sum over the selection)
    routed_scale  sigmoid gate: the routed scaling factor
    selection_bias  sigmoid gate: float32 CUDA tensor [E] or None
    cache_policy  slot cache replacement: "lfu" (default) or "lru"
    bits          width of the expert weight codes: 4 (default) or 2
    """

    def __init__(self, hidden: int, n_experts: int, inter: int, top_k: int, shared_inter: int,
                 router_q: torch.Tensor, router_scale: torch.Tensor,
                 experts: torch.Tensor | None, shared: torch.Tensor | None, act: str = "bf16",
                 n_slots: int = 0, host_pool: torch.Tensor | None = None,
                 slots: torch.Tensor | None = None, gate: str = "softmax",
                 routed_scale: float = 1.0, selection_bias: torch.Tensor | None = None,
                 cache_policy: str = "lfu", bits: int = 4):
        self.hidden, self.n_experts, self.inter = hidden, n_experts, inter
        self.bits = bits
        self.top_k, self.shared_inter, self.act = top_k, shared_inter, act
        self.n_slots = n_slots
        if gate not in ("softmax", "sigmoid"):
            raise ValueError("gate must be 'softmax' or 'sigmoid'")
        self.gate = gate
        self._keep = (router_q, router_scale, experts, shared, host_pool, slots, selection_bias)
        d = Desc(hidden, n_experts, inter, top_k, shared_inter, 64,
                 MOE_BF16 if act == "bf16" else MOE_F32,
                 MOE_SIGMOID_TOPK if gate == "sigmoid" else MOE_SOFTMAX_TOPK, n_slots,
                 float(routed_scale), {"lfu": MOE_CACHE_LFU, "lru": MOE_CACHE_LRU}[cache_policy], bits)
        hp = None
        if host_pool is not None:
            if host_pool.is_cuda or not host_pool.is_pinned() or not host_pool.is_contiguous():
                raise ValueError("host_pool must be a contiguous pinned CPU tensor")
            hp = host_pool.data_ptr()
        w = Weights(_dev(router_q, "router_q", torch.int8),
                    _dev(router_scale, "router_scale"),
                    None if experts is None else _dev(experts, "experts", torch.uint8),
                    None if shared is None else _dev(shared, "shared", torch.uint8), hp,
                    None if slots is None else _dev(slots, "slots", torch.uint8),
                    None if selection_bias is None else _dev(selection_bias, "selection_bias", torch.float32))
        h = C.c_void_p()
        _check(lib().moe_layer_create(C.byref(d), C.byref(w), C.byref(h)))
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _LIB is not None:
            _LIB.moe_layer_destroy(h)
            self.handle = None

    @property
    def act_dtype(self):
        return torch.bfloat16 if self.act == "bf16" else torch.float32

    def workspace_bytes(self, n_tokens: int) -> int:
        return int(lib().moe_workspace_bytes(self.handle, n_tokens))

    def workspace(self, n_tokens: int) -> torch.Tensor:
        return torch.zeros(self.workspace_bytes(n_tokens), dtype=torch.uint8, device="cuda")

    def _x(self, x: torch.Tensor) -> int:
        if x.dim() != 2 or x.shape[1] != self.hidden:
            raise ValueError(f"x must be [T][{self.hidden}]")
        return _dev(x, "x", self.act_dtype)

    def route(self, x: torch.Tensor, ws: torch.Tensor | None = None, out=None):
        T = x.shape[0]
        ws = self.workspace(T) if ws is None else ws
        if out is None:
            ids = torch.empty(T, self.top_k, dtype=torch.int32, device="cuda")
            w = torch.empty(T, self.top_k, dtype=torch.float32, device="cuda")
        else:
            ids, w = out
            if ids.shape != (T, self.top_k) or w.shape != (T, self.top_k):
                raise ValueError("out must be ([T][k] int32, [T][k] float32)")
        _check(lib().moe_route_topk(self.handle, self._x(x), T, _dev(ids, "ids", torch.int32),
                                    _dev(w, "w", torch.float32), _dev(ws, "workspace"), _stream()))
        return ids, w

    def ffn(self, x: torch.Tensor, ids: torch.Tensor, ws: torch.Tensor | None = None):
        T = x.shape[0]
        ws = self.workspace(T) if ws is None else ws
        eo = torch.empty(T, self.top_k + 1, self.hidden, dtype=torch.float32, device="cuda")
        _check(lib().moe_expert_ffn(self.handle, self._x(x), T, _dev(ids, "ids", torch.int32),
                                    _dev(ws, "workspace"), eo.data_ptr(), _stream()))
        return eo

    def combine(self, eo: torch.Tensor, w: torch.Tensor, y_dtype=torch.float32):
        T = eo.shape[0]
        y = torch.empty(T, self.hidden, dtype=y_dtype, device="cuda")
        code = MOE_BF16 if y_dtype == torch.bfloat16 else MOE_F32
        _check(lib().moe_combine(self.handle, _dev(eo, "expert_out", torch.float32),
                                 _dev(w, "w", torch.float32), T, y.data_ptr(), code, _stream()))
        return y

    def forward(self, x: torch.Tensor, ws: torch.Tensor | None = None, out=None):
        T = x.shape[0]
        ws = self.workspace(T) if ws is None else ws
        if out is None:
            ids = torch.empty(T, self.top_k, dtype=torch.int32, device="cuda")
            w = torch.empty(T, self.top_k, dtype=torch.float32, device="cuda")
            y = torch.empty(T, self.hidden, dtype=torch.float32, device="cuda")
        else:
            ids, w, y = out
        _check(lib().moe_layer_forward(self.handle, self._x(x), T, _dev(ids, "ids", torch.int32),
                                       _dev(w, "w", torch.float32), _dev(y, "y", torch.float32),
                                       _dev(ws, "workspace"), _stream()))
        return ids, w, y

    def forward_noalloc(self, x: torch.Tensor, out):
        """forward() with the library's static scratch as the workspace
        (moe_layer_forward_noalloc): out = (ids, w, y) preallocated by the caller."""
        T = x.shape[0]
        ids, w, y = out
        _check(lib().moe_layer_forward_noalloc(self.handle, self._x(x), T, _dev(ids, "ids", torch.int32),
                                               _dev(w, "w", torch.float32), _dev(y, "y", torch.float32),
                                               _stream()))
        return ids, w, y

    def cache_stats(self):
        h, m = C.c_uint64(), C.c_uint64()
        _check(lib().moe_cache_stats(self.handle, C.byref(h), C.byref(m)))
        return int(h.value), int(m.value)

    def cache_pin(self, experts) -> None:
        """Pin these expert ids into the slot cache (replacing any pinned set)."""
        ids = (C.c_int32 * max(len(experts), 1))(*[int(e) for e in experts])
        _check(lib().moe_cache_pin(self.handle, ids, len(experts), _stream()))

    def cache_usage(self) -> list[int]:
        """The per-expert selection counts (the usage heatmap), [E]."""
        out = (C.c_uint64 * self.n_experts)()
        _check(lib().moe_cache_usage(self.handle, out))
        return [int(v) for v in out]

    def cache_pin_hottest(self, n: int, counts=None) -> None:
        """Pin the n experts with the largest counts (a saved heatmap of E
        non-negative integers, or this layer's own when counts is None), ties
        to the lower id."""
        arr = None
        if counts is not None:
            vals = [int(v) for v in counts]
            if len(vals) != self.n_experts or min(vals) < 0:
                raise ValueError(f"counts must be {self.n_experts} non-negative integers")
            arr = (C.c_uint64 * self.n_experts)(*vals)
        _check(lib().moe_cache_pin_hottest(self.handle, arr, int(n), _stream()))

    def cache_prefetch(self, x_hint: torch.Tensor, n_predict: int | None = None,
                       ws: torch.Tensor | None = None) -> list[int]:
        """Router lookahead: fetch the experts x_hint ([H] or [1][H]) selects into
        the slot cache ahead of this layer's own call; returns the predicted ids."""
        n = self.top_k if n_predict is None else int(n_predict)
        ws = self.workspace(1) if ws is None else ws
        out = (C.c_int32 * max(n, 1))()
        _check(lib().moe_cache_prefetch(self.handle, self._x(x_hint.reshape(1, -1)), n,
                                        _dev(ws, "workspace"), out, _stream()))
        return [int(v) for v in out[:n]]

    def cache_prefetch_ids(self, experts) -> None:
        """Prefetch these host-side predicted expert ids (no router, no wait)."""
        ids = (C.c_int32 * max(len(experts), 1))(*[int(e) for e in experts])
        _check(lib().moe_cache_prefetch_ids(self.handle, ids, len(experts), _stream()))

    def prefetch_stats(self):
        """(copies issued by cache_prefetch, prefetched experts selected before eviction)."""
        a, b = C.c_uint64(), C.c_uint64()
        _check(lib().moe_cache_prefetch_stats(self.handle, C.byref(a), C.byref(b)))
        return int(a.value), int(b.value)

    def poll_error(self, ws: torch.Tensor):
        _check(lib().moe_poll_device_error(self.handle, _dev(ws, "workspace"), _stream()))


def stack_forward(layers: list[Layer], x: torch.Tensor, ws: torch.Tensor, out=None):
    """x [L][T][H] -> (ids [L][T][k], w [L][T][k], y [L][T][H]); layer l reads x[l]."""
    L, T, H = x.shape
    k = layers[0].top_k
    if len(layers) != L:
        raise ValueError(f"x holds {L} layers' inputs for {len(layers)} layers")
    for lay in layers:
        if lay.hidden != H or lay.top_k != k or lay.act != layers[0].act:
            raise ValueError("stack layers must share hidden, top_k and activation dtype")
    if out is None:
        ids = torch.empty(L, T, k, dtype=torch.int32, device="cuda")
        w = torch.empty(L, T, k, dtype=torch.float32, device="cuda")
        y = torch.empty(L, T, H, dtype=torch.float32, device="cuda")
    else:
        ids, w, y = out
    arr = (C.c_void_p * L)(*[l.handle.value for l in layers])
    _check(lib().moe_stack_forward(arr, L, _dev(x, "x", layers[0].act_dtype), T * H, T,
                                   _dev(ids, "ids", torch.int32), _dev(w, "w", torch.float32),
                                   _dev(y, "y", torch.float32), T * H, _dev(ws, "workspace"),
                                   _stream()))
    return ids, w, y


def stream_read(buf: torch.Tensor, offset: int, nbytes: int, n_blocks: int, sink: torch.Tensor) -> None:
    """Plain streaming read of nbytes of the uint8 CUDA tensor buf from byte
    offset (moe_stream_read): the measured HBM reference."""
    if offset < 0 or offset + nbytes > buf.numel() * buf.element_size():
        raise ValueError("read past the end of buf")
    _check(lib().moe_stream_read(_dev(buf, "buf") + offset, nbytes, n_blocks,
                                 _dev(sink, "sink", torch.int32), _stream()))


class KernelTimer:
    """Per-launch hipEvent timing of every library kernel (moe_profile_*)."""

    def __init__(self, capacity: int = 65536):
        self.capacity = capacity

    def __enter__(self):
        _check(lib().moe_profile_start(self.capacity))
        return self

    def __exit__(self, *exc):
        _check(lib().moe_profile_stop())

    def read(self):
        import numpy as np
        ids = np.zeros(self.capacity, dtype=np.int32)
        ms = np.zeros(self.capacity, dtype=np.float32)
        n = lib().moe_profile_read(ids.ctypes.data, ms.ctypes.data, self.capacity)
        if n < 0:
            _check(n)
        return [(KERNEL_NAMES[int(i)], float(m)) for i, m in zip(ids[:n], ms[:n])]
