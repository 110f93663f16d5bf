"""The C ABI without a GPU: the library loads, exports every function declared
in include/moe_layer.h, and rejects bad descriptors on the host before any HIP
call."""
import ctypes as C
import os
import re

import pytest

from bit_routed_expert_moe_amd import layer as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_layer.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_record_bytes_formula():
    lib = L.lib()
    for H, I in [(64, 64), (256, 128), (2816, 704), (6144, 2048)]:
        assert lib.moe_expert_record_bytes(H, I) == 27 * H * I // 16
    for H, I in [(0, 64), (64, 0), (100, 64), (64, 96), (-64, 64)]:
        assert lib.moe_expert_record_bytes(H, I) == 0


def test_record_bytes_by_bit_width():
    # codes at bits/8 bytes per weight, plus 4 bytes of (scale, bias) per 64 weights
    lib = L.lib()
    for H, I in [(64, 64), (256, 128), (2816, 704), (6144, 2048)]:
        assert lib.moe_expert_record_bytes_bits(H, I, 4) == 3 * H * I // 2 + 3 * H * I // 16
        assert lib.moe_expert_record_bytes_bits(H, I, 2) == 3 * H * I // 4 + 3 * H * I // 16
        assert L.record_bytes(H, I, 2) == 15 * H * I // 16
    for bits in (0, 1, 3, 8):
        assert lib.moe_expert_record_bytes_bits(256, 128, bits) == 0
    assert lib.moe_expert_record_bytes_bits(100, 64, 2) == 0


def test_status_strings():
    lib = L.lib()
    for code, name in L.STATUS.items():
        assert lib.moe_status_str(code).decode() == name


def _create(desc, weights):
    h = C.c_void_p()
    st = L.lib().moe_layer_create(C.byref(desc), C.byref(weights), C.byref(h))
    return st, L.lib().moe_last_error().decode()


GOOD = dict(hidden=256, n_experts=32, inter=128, top_k=8, shared_inter=256, group=64,
            act_dtype=1, gate_fn=0, n_slots=0)
FAKE = dict(router_q=0x10000, router_scale=0x20000, experts=0x30000, shared=0x40000)


@pytest.mark.parametrize("change,status", [
    (dict(group=32), -2), (dict(hidden=100), -2), (dict(hidden=0), -2), (dict(hidden=16384), -2),
    (dict(inter=96), -2), (dict(shared_inter=100), -2), (dict(n_experts=0), -2),
    (dict(n_experts=2048), -2), (dict(top_k=0), -2), (dict(top_k=33), -2),
    (dict(n_experts=4, top_k=5), -2), (dict(act_dtype=7), -1), (dict(gate_fn=2), -1),
    (dict(routed_scale=2.5), -1), (dict(gate_fn=1, routed_scale=-1.0), -1),
    (dict(gate_fn=1, routed_scale=float("nan")), -1), (dict(gate_fn=1, routed_scale=float("inf")), -1),
    (dict(cache_policy=2), -1), (dict(cache_policy=1), -1),  # LRU needs a slot cache
    (dict(n_slots=4), -2), (dict(n_slots=16), -1), (dict(n_slots=-1), -2),
    (dict(bits=3), -1), (dict(bits=8), -1), (dict(bits=-2), -1),
])
def test_create_rejects_bad_descriptor(change, status):
    d = L.Desc(**{**GOOD, **change})
    w = L.Weights(**FAKE)
    st, msg = _create(d, w)
    assert st == status, msg
    assert msg


def test_create_rejects_missing_and_misaligned_pointers():
    d = L.Desc(**GOOD)
    assert _create(d, L.Weights(**{**FAKE, "experts": None}))[0] == -1
    assert _create(d, L.Weights(**{**FAKE, "shared": None}))[0] == -1
    d0 = L.Desc(**{**GOOD, "shared_inter": 0})
    assert _create(d0, L.Weights(**FAKE))[0] == -1            # shared given but size 0
    assert _create(d, L.Weights(**{**FAKE, "experts": 0x30008}))[0] == -3
    assert _create(d, L.Weights(**{**FAKE, "router_q": 0x10004}))[0] == -3
    assert _create(d, L.Weights(**{**FAKE, "host_pool": 0x50000}))[0] == -1
    # the selection bias belongs to the sigmoid gate and must be 4-byte aligned
    assert _create(d, L.Weights(**{**FAKE, "selection_bias": 0x60000}))[0] == -1
    ds = L.Desc(**{**GOOD, "gate_fn": 1, "routed_scale": 2.5})
    assert _create(ds, L.Weights(**{**FAKE, "selection_bias": 0x60002}))[0] == -3


def test_null_handles():
    lib = L.lib()
    assert lib.moe_cache_pin(None, None, 0, None) == -1
    assert lib.moe_cache_pin_hottest(None, None, 0, None) == -1
    counts = (C.c_uint64 * 4)()
    assert lib.moe_cache_usage(None, counts) == -1
    assert lib.moe_cache_prefetch(None, None, 8, None, None, None) == -1
    assert lib.moe_cache_prefetch_ids(None, None, 1, None) == -1
    a, b = C.c_uint64(), C.c_uint64()
    assert lib.moe_cache_prefetch_stats(None, C.byref(a), C.byref(b)) == -1
    assert lib.moe_layer_destroy(None) == -1
    assert lib.moe_workspace_bytes(None, 1) == 0
    assert lib.moe_layer_forward(None, None, 1, None, None, None, None, None) == -1
    assert lib.moe_stack_forward(None, 0, None, 0, 1, None, None, None, 0, None, None) == -1


def test_stream_read_rejects_bad_arguments_on_the_host():
    lib = L.lib()
    assert lib.moe_stream_read(None, 16, 1, 0x20000, None) == -1
    assert lib.moe_stream_read(0x10000, 0, 1, 0x20000, None) == -1
    assert lib.moe_stream_read(0x10000, 24, 1, 0x20000, None) == -1   # not whole 16-byte vectors
    assert lib.moe_stream_read(0x10000, 16, 0, 0x20000, None) == -1
    assert lib.moe_stream_read(0x10008, 16, 1, 0x20000, None) == -3
