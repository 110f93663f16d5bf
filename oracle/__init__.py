"""CPU oracle for the routed-expert MoE layer -- TEST INFRASTRUCTURE.

Only tests/, ``__graft_entry__.smoke()`` and bench.py's ``cpu_baseline`` leg
may import this package.  The GPU library never calls it and shares no code
with it.  All arithmetic lives in ``moe_oracle.c`` (IEEE double, plain loops);
this module only moves numpy arrays in and out through ctypes.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "libmoe_oracle.so")

_dp = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_i8p = np.ctypeslib.ndpointer(dtype=np.int8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")


def _opt(ptr_type):
    """ndpointer that also accepts None (a NULL argument)."""
    class _Opt(ptr_type):
        @classmethod
        def from_param(cls, obj):
            return None if obj is None else ptr_type.from_param(obj)
    return _Opt


class Oracle:
    def __init__(self, lib_path: str = DEFAULT_LIB):
        if not os.path.exists(lib_path):
            from . import build as _b
            _b.build(out=lib_path)
        self.lib = L = C.CDLL(lib_path)
        self.path = lib_path
        L.oracle_set_threads.argtypes = [C.c_int]
        L.oracle_set_threads.restype = C.c_int
        L.oracle_f16_to_f64.argtypes = [C.c_uint16]
        L.oracle_f16_to_f64.restype = C.c_double
        L.oracle_bf16_to_f64.argtypes = [C.c_uint16]
        L.oracle_bf16_to_f64.restype = C.c_double
        L.oracle_act_to_f64.argtypes = [C.c_int, C.c_void_p, C.c_int64, _dp]
        L.oracle_record_bytes.argtypes = [C.c_int, C.c_int]
        L.oracle_record_bytes.restype = C.c_size_t
        L.oracle_record_bytes_bits.argtypes = [C.c_int, C.c_int, C.c_int]
        L.oracle_record_bytes_bits.restype = C.c_size_t
        L.oracle_dequant_record.argtypes = [C.c_int, C.c_int, _u8p, _dp, _dp, _dp]
        L.oracle_dequant_record_bits.argtypes = [C.c_int, C.c_int, C.c_int, _u8p, _dp, _dp, _dp]
        L.oracle_router_logits.argtypes = [C.c_int, C.c_int, _i8p, _u16p, _dp, _dp]
        L.oracle_select_topk.argtypes = [C.c_int, C.c_int, _dp, _i32p]
        L.oracle_softmax_gates.argtypes = [C.c_int, _dp, _dp]
        L.oracle_sigmoid_route.argtypes = [C.c_int, C.c_int, _dp, _opt(_dp), C.c_double, _i32p, _dp]
        L.oracle_silu.argtypes = [C.c_double]
        L.oracle_silu.restype = C.c_double
        L.oracle_expert_ffn.argtypes = [C.c_int, C.c_int, _u8p, _dp, _dp,
                                        _opt(_dp), _opt(_dp), _opt(_dp)]
        L.oracle_expert_ffn_bits.argtypes = [C.c_int, C.c_int, C.c_int, _u8p, _dp, _dp,
                                             _opt(_dp), _opt(_dp), _opt(_dp)]
        L.oracle_combine.argtypes = [C.c_int, C.c_int, _dp, _dp, _opt(_dp), _dp]
        L.oracle_layer_token.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int,
                                         _i8p, _u16p, _u8p, _opt(_u8p), _dp, _i32p, _dp,
                                         _dp, _opt(_dp)]

    # -- plumbing ----------------------------------------------------------
    def set_threads(self, n: int) -> int:
        return int(self.lib.oracle_set_threads(int(n)))

    def f16(self, bits: int) -> float:
        return self.lib.oracle_f16_to_f64(int(bits))

    def bf16(self, bits: int) -> float:
        return self.lib.oracle_bf16_to_f64(int(bits))

    def act_to_f64(self, act: str, x: np.ndarray) -> np.ndarray:
        if act == "f32":
            src = np.ascontiguousarray(x, dtype=np.float32)
            code = 0
        elif act == "bf16":
            src = np.ascontiguousarray(x, dtype=np.uint16)
            code = 1
        else:
            raise ValueError(act)
        out = np.empty(src.shape, dtype=np.float64)
        self.lib.oracle_act_to_f64(code, src.ctypes.data, src.size, out)
        return out

    def record_bytes(self, H: int, I: int, bits: int = 4) -> int:
        if bits == 4:
            return int(self.lib.oracle_record_bytes(H, I))
        return int(self.lib.oracle_record_bytes_bits(bits, H, I))

    # -- the method --------------------------------------------------------
    def dequant_record(self, H: int, I: int, rec: np.ndarray, bits: int = 4):
        G = np.empty((I, H)); U = np.empty((I, H)); D = np.empty((H, I))
        r = np.ascontiguousarray(rec, dtype=np.uint8)
        if bits == 4:
            self.lib.oracle_dequant_record(H, I, r, G, U, D)
        else:
            self.lib.oracle_dequant_record_bits(bits, H, I, r, G, U, D)
        return G, U, D

    def router_logits(self, rq: np.ndarray, rs: np.ndarray, x: np.ndarray) -> np.ndarray:
        E, H = rq.shape
        out = np.empty(E)
        self.lib.oracle_router_logits(H, E, np.ascontiguousarray(rq, dtype=np.int8),
                                      np.ascontiguousarray(rs, dtype=np.uint16),
                                      np.ascontiguousarray(x, dtype=np.float64), out)
        return out

    def select_topk(self, logits: np.ndarray, k: int) -> np.ndarray:
        ids = np.empty(k, dtype=np.int32)
        lg = np.ascontiguousarray(logits, dtype=np.float64)
        self.lib.oracle_select_topk(lg.size, k, lg, ids)
        return ids

    def softmax_gates(self, sel_logits: np.ndarray) -> np.ndarray:
        sl = np.ascontiguousarray(sel_logits, dtype=np.float64)
        w = np.empty(sl.size)
        self.lib.oracle_softmax_gates(sl.size, sl, w)
        return w

    def silu(self, v: float) -> float:
        return self.lib.oracle_silu(float(v))

    def expert_ffn(self, H: int, I: int, rec: np.ndarray, x: np.ndarray,
                   intermediates: bool = False, bits: int = 4):
        y = np.empty(H)
        g = np.empty(I) if intermediates else None
        u = np.empty(I) if intermediates else None
        h = np.empty(I) if intermediates else None
        r = np.ascontiguousarray(rec, dtype=np.uint8)
        xx = np.ascontiguousarray(x, dtype=np.float64)
        if bits == 4:
            self.lib.oracle_expert_ffn(H, I, r, xx, y, g, u, h)
        else:
            self.lib.oracle_expert_ffn_bits(bits, H, I, r, xx, y, g, u, h)
        return (y, g, u, h) if intermediates else y

    def combine(self, w: np.ndarray, y_routed: np.ndarray, y_shared: np.ndarray | None):
        k, H = y_routed.shape
        y = np.empty(H)
        self.lib.oracle_combine(k, H, np.ascontiguousarray(w, dtype=np.float64),
                                np.ascontiguousarray(y_routed, dtype=np.float64),
                                None if y_shared is None else
                                np.ascontiguousarray(y_shared, dtype=np.float64), y)
        return y

    def layer_token(self, rq, rs, pool: np.ndarray, shared: np.ndarray | None, I: int,
                    I_shared: int, k: int, x: np.ndarray):
        """Whole layer for one token with every routed record in ``pool``
        (E records back to back).  Returns ids, w, y, logits."""
        E, H = rq.shape
        ids = np.empty(k, dtype=np.int32)
        w = np.empty(k); y = np.empty(H); lg = np.empty(E)
        self.lib.oracle_layer_token(H, E, I, k, I_shared,
                                    np.ascontiguousarray(rq, dtype=np.int8),
                                    np.ascontiguousarray(rs, dtype=np.uint16),
                                    np.ascontiguousarray(pool, dtype=np.uint8),
                                    None if shared is None else
                                    np.ascontiguousarray(shared, dtype=np.uint8),
                                    np.ascontiguousarray(x, dtype=np.float64), ids, w, y, lg)
        return ids, w, y, lg

    def sigmoid_route(self, logits: np.ndarray, k: int, bias: np.ndarray | None = None,
                      scale: float = 1.0):
        """Sigmoid scores, top-k of score + bias, gates = scale * score / sum."""
        lg = np.ascontiguousarray(logits, dtype=np.float64)
        ids = np.empty(k, dtype=np.int32)
        w = np.empty(k)
        self.lib.oracle_sigmoid_route(lg.size, k, lg, None if bias is None else
                                      np.ascontiguousarray(bias, dtype=np.float64), float(scale), ids, w)
        return ids, w

    def route(self, rq, rs, x: np.ndarray, k: int, gate: str = "softmax",
              bias: np.ndarray | None = None, scale: float = 1.0):
        """Router, exact top-k and gates for one token: softmax over the
        selected logits, or the sigmoid router (selection bias, scale)."""
        lg = self.router_logits(rq, rs, x)
        if gate == "sigmoid":
            ids, w = self.sigmoid_route(lg, k, bias, scale)
            return ids, w, lg
        ids = self.select_topk(lg, k)
        return ids, self.softmax_gates(lg[ids]), lg


_DEFAULT: Oracle | None = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
