"""Plant plausible mistakes in copies of the oracle and check a pin catches each.

Each mutant is a textual edit of oracle/moe_oracle.c compiled into a temporary
library; the real oracle is untouched.  A mutant that passes every pin would
mean the pins cannot tell that mistake from the right answer.
"""
import os
import tempfile

import pytest

import oracle
import oracle.build as ob
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")

MUTANTS = {
    "nibble_order_swapped": ("return (elem & 1) ? (byte >> 4) : (byte & 0x0F);",
                             "return (elem & 1) ? (byte & 0x0F) : (byte >> 4);"),
    "gate_up_rows_swapped": ("int b = i / 32, r = i % 32 + 32 * which, g = k / 64, c = (k % 64) / 32, e = k % 32;",
                             "int b = i / 32, r = i % 32 + 32 * (1 - which), g = k / 64, c = (k % 64) / 32, e = k % 32;"),
    "chunk_stride": ("(size_t)c * 1024", "(size_t)c * 512"),
    "down_bias_dropped": ("acc += (s * q_d(bits, rec, H, I, o, i) + bias) * h[i];",
                          "acc += (s * q_d(bits, rec, H, I, o, i)) * h[i];"),
    "silu_sign": ("return v / (1.0 + exp(-v));", "return v / (1.0 + exp(v));"),
    "gate_up_roles_swapped": ("h[i] = oracle_silu(g) * u;", "h[i] = oracle_silu(u) * g;"),
    "topk_tie_breaks_high_id": ("logits[e] > logits[best]", "logits[e] >= logits[best]"),
    "gates_not_normalised": ("w[j] /= z;", "w[j] /= (double)k;"),
    "router_scale_dropped": ("logits[e] = oracle_f16_to_f64(rs[e]) * acc;", "logits[e] = acc;"),
    "f16_subnormal_exponent": ("v = ldexp((double)mant, -24);", "v = ldexp((double)mant, -25);"),
    "gu_sb_block_pairs_shared": ("gu_segment(bits, H, b, h) + seg_codes(bits)",
                                 "gu_segment(bits, H, b & ~1, h) + seg_codes(bits)"),
    "gu_sb_group_ignored": ("gu_segment(bits, H, b, h) + seg_codes(bits)",
                            "gu_segment(bits, H, b, 0) + seg_codes(bits)"),
    "gu_sb_row_stride": ("seg_codes(bits) + (size_t)r * 4", "seg_codes(bits) + (size_t)(r / 2) * 4"),
    "down_sb_group_ignored": ("d_segment(bits, H, I, o / 64, g)", "d_segment(bits, H, I, o / 64, 0)"),
    "down_row_stride": ("d_segment(4, H, I, t, g) + (size_t)c * 1024 + (size_t)r * 16",
                        "d_segment(4, H, I, t, g) + (size_t)c * 1024 + (size_t)r * 8"),
    "down_tile_ignored": ("size_t off = d_segment(4, H, I, t, g)", "size_t off = d_segment(4, H, I, 0, g)"),
    "down_part_offset": ("return ((size_t)(I / 32) * (H / 64) + (size_t)t * (I / 64) + g) * seg_bytes(bits);",
                         "return ((size_t)(I / 64) * (H / 64) + (size_t)t * (I / 64) + g) * seg_bytes(bits);"),
    "shared_dropped": ("acc += y_shared[o];", "acc += 0.0 * y_shared[o];"),
    "bf16_shift": ("(uint32_t)b << 16", "(uint32_t)b << 15"),
    "crumb_order_reversed": ("return (rec[byte_off] >> (2 * (elem & 3))) & 3;",
                             "return (rec[byte_off] >> (6 - 2 * (elem & 3))) & 3;"),
    "two_bit_chunk_width": ("g = k / 64, e = k % 64;\n    size_t off = gu_segment(2",
                            "g = k / 32, e = k % 32;\n    size_t off = gu_segment(2"),
    "two_bit_down_stride": ("d_segment(2, H, I, t, g) + (size_t)r * 16 + e / 4",
                            "d_segment(2, H, I, t, g) + (size_t)r * 8 + e / 4"),
    "two_bit_down_tile_ignored": ("size_t off = d_segment(2, H, I, t, g)", "size_t off = d_segment(2, H, I, 0, g)"),
    "sigmoid_gates_use_bias": ("w[j] = 1.0 / (1.0 + exp(-logits[ids[j]]));",
                               "w[j] = key[ids[j]];"),
    "sigmoid_scale_dropped": ("w[j] = scale * (w[j] / z);", "w[j] = w[j] / z;"),
    "sigmoid_bias_ignored": ("+ (bias ? bias[e] : 0.0);", "+ 0.0;"),
    "sigmoid_sign": ("key[e] = 1.0 / (1.0 + exp(-logits[e]))", "key[e] = 1.0 / (1.0 + exp(logits[e]))"),
}


@pytest.fixture(scope="module")
def src_text():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, src_text, tmp_path):
    old, new = MUTANTS[name]
    assert src_text.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src_text.replace(old, new)
    src = tmp_path / "mut.c"
    src.write_text(mutated)
    lib = ob.build(src=str(src), out=str(tmp_path / "libmut.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {name}"
