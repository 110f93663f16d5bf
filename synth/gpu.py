"""GPU fill of synthetic expert records (same definition as synth.expert_record)."""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_synth.so")
_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        _LIB = C.CDLL(LIB_PATH)
        _LIB.synth_fill_records.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_int, C.c_uint64,
                                            C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_int]
        _LIB.synth_fill_records.restype = C.c_int
    return _LIB


def fill_records(dst: torch.Tensor, hidden: int, inter: int, seed: int, layer: int,
                 first_index: int, n_records: int, stride: int | None = None, bits: int = 4):
    """Writes n_records records (experts first_index.., or the shared expert when
    first_index < 0) into the uint8 CUDA tensor dst, back to back."""
    from . import record_bytes
    rb = record_bytes(hidden, inter, bits)
    stride = rb if stride is None else stride
    assert dst.is_cuda and dst.dtype == torch.uint8 and dst.is_contiguous()
    assert dst.numel() >= stride * (n_records - 1) + rb
    done = 0
    while done < n_records:
        n = min(65535, n_records - done)
        st = _lib().synth_fill_records(dst.data_ptr() + done * stride, stride, hidden, inter,
                                       seed, layer, -1 if first_index < 0 else first_index + done,
                                       n, torch.cuda.current_stream().cuda_stream, bits)
        if st != 0:
            raise RuntimeError(f"synth_fill_records failed ({st})")
        done += n
