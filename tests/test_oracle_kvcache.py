"""Pins for the KV-append oracle and its INT8 / INT4 encoders (CPU only).

Hand-derived rows pin round-half-to-even, the scale and zero-point formulas,
the clamp, the degenerate all-equal rows and the nibble order; the round
trip through the independent decoders (oracle/quant.py) bounds the error by
half a quantisation step; the torch test-data encoders of the workloads
module, written separately from the same reading, must agree bit for bit;
and the slot arithmetic of append_kv is checked on a hand-built pool.
"""
import numpy as np
import pytest
import torch

from decode_attention_paged_gqa_amd import workloads as W
from oracle import kvcache as OK
from oracle import quant as OQ


# ---- INT8: s = fp16(max|x| / 127) (1 if 0), code = clamp(rne(x / s), -127, 127)
@pytest.mark.parametrize("x,s,codes", [
    # amax 127 -> s = 1; 2.5 rounds to the even 2
    ([0.0, 1.0, -1.0, 2.5, 127.0], 1.0, [0, 1, -1, 2, 127]),
    # amax 254 -> s = 2; x / s = 127, -1.5, 0.75, -0.25 -> 127, -2, 1, 0
    ([254.0, -3.0, 1.5, -0.5], 2.0, [127, -2, 1, 0]),
    # all zero: fp16(0) -> s = 1
    ([0.0, 0.0, 0.0], 1.0, [0, 0, 0]),
    # amax / 127 underflows fp16 to 0 -> s = 1, codes rne(x) = 0
    ([1e-9, -1e-9], 1.0, [0, 0]),
])
def test_int8_hand_rows(x, s, codes):
    c, sc = OK.quantize_int8(np.array(x, dtype=np.float32))
    assert float(sc) == s
    np.testing.assert_array_equal(c, np.array(codes, dtype=np.int8))


def _int4_hand_row():
    """Three 32-groups, each value and code derived by hand:
    group 0: min -3, max 27 -> s = 30/15 = 2; z = rne(3/2 = 1.5) = 2 (half to even);
             x/2 = -1.5, 13.5, 0.5, -0.5, 1.5, 2.5, 0.25, 0 -> rne -2, 14, 0, -0, 2, 2, 0, 0
             -> + z = 0, 16 (clamp 15), 2, 2, 4, 4, 2, 2 (rest 0 -> 2)
    group 1: all 3 -> range 0 -> s = 1; z = clamp(rne(-3), 0, 15) = 0; nib = 3
    group 2: all -3 -> s = 1; z = 3; nib = clamp(-3 + 3) = 0
    """
    g0 = np.zeros(32, dtype=np.float32)
    g0[:7] = [-3.0, 27.0, 1.0, -1.0, 3.0, 5.0, 0.5]
    x = np.concatenate([g0, np.full(32, 3.0, np.float32), np.full(32, -3.0, np.float32)])
    nib0 = np.full(32, 2)
    nib0[:6] = [0, 15, 2, 2, 4, 4]
    nib = np.concatenate([nib0, np.full(32, 3), np.zeros(32, int)])
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)
    sz = np.array([[2.0, 2.0], [1.0, 0.0], [1.0, 3.0]], dtype=np.float16)
    return x, packed, sz


def test_int4_hand_row_rounding_zero_clamp_and_nibble_order():
    x, packed, sz = _int4_hand_row()
    p, s = OK.quantize_int4(x)
    assert p[0] == 0xF0 and p[1] == 0x22 and p[2] == 0x44  # elem 2j low, 2j+1 high
    np.testing.assert_array_equal(p, packed)
    np.testing.assert_array_equal(s, sz)


def test_int4_zero_point_zero_is_stored_as_plus_zero():
    # min = 0.01, s ~ 0.1993: -min / s = -0.05 rounds to -0 -> the code 0 is stored as +0
    x = np.linspace(0.01, 3.0, 32, dtype=np.float32)
    _, sz = OK.quantize_int4(x)
    assert sz[0, 1].view(np.uint16) == 0


def test_int4_all_equal_groups_decode_exactly():
    x, _, _ = _int4_hand_row()
    p, s = OK.quantize_int4(x)
    xh = OQ.dequant_int4(p, s.view(np.uint16))
    np.testing.assert_array_equal(xh[32:], x[32:].astype(np.float64))


def _bf16_rows(seed, shape=(64, 8, 128)):
    return torch.randn(shape, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)


def test_int8_roundtrip_within_half_step():
    x = _bf16_rows(0).float().numpy()
    c, s = OK.quantize_int8(x)
    xh = OQ.dequant_int8(c, s.view(np.uint16))
    sf = s.astype(np.float64)[..., None]
    inside = np.abs(x / sf) <= 127
    assert inside.mean() > 0.99
    assert np.all((np.abs(x - xh) <= sf * (0.5 + 1e-6))[inside])


def test_int4_roundtrip_within_half_step():
    x = _bf16_rows(1).float().numpy()
    p, sz = OK.quantize_int4(x)
    xh = OQ.dequant_int4(p, sz.view(np.uint16))
    s = np.repeat(sz[..., 0].astype(np.float64), 32, axis=-1)
    z = np.repeat(sz[..., 1].astype(np.float64), 32, axis=-1)
    q = x / s + z
    inside = (q >= -0.5) & (q <= 15.5)
    assert inside.mean() > 0.99
    assert np.all((np.abs(x - xh) <= s * (0.5 + 1e-6))[inside])


def test_encoders_match_the_torch_test_data_encoders_bit_for_bit():
    x = _bf16_rows(2)
    c, s = OK.quantize_int8(x.float().numpy())
    ct, st = W.quantize_int8(x)
    np.testing.assert_array_equal(c, ct.numpy())
    np.testing.assert_array_equal(s.view(np.uint16), W.host_u16(st))
    p, sz = OK.quantize_int4(x.float().numpy())
    pt, szt = W.quantize_int4(x)
    np.testing.assert_array_equal(p, pt.numpy())
    np.testing.assert_array_equal(sz.view(np.uint16), W.host_u16(szt))


def test_append_writes_only_valid_slots_at_page_and_offset():
    # P = 3 pages of 4 slots; slots 5 -> (page 1, offset 1), 10 -> (2, 2);
    # -1 (sentinel) and 12 (= P * page_size, past the pool) write nothing
    pool = np.zeros((3, 4, 1, 2))
    new = np.arange(1, 9, dtype=np.float64).reshape(4, 1, 2)
    OK.append_kv(pool, new, [5, -1, 10, 12], 4, "dense")
    want = np.zeros((3, 4, 1, 2))
    want[1, 1] = new[0]
    want[2, 2] = new[2]
    np.testing.assert_array_equal(pool, want)


def test_append_quantises_each_row_with_its_encoder():
    x = _bf16_rows(3, (3, 2, 128)).float().numpy()
    codes = np.zeros((2, 16, 2, 128), np.int8)
    scale = np.zeros((2, 16, 2), np.float16)
    OK.append_kv(codes, x, [17, 0, 31], 16, "int8", scale)
    for n, slot in enumerate([17, 0, 31]):
        c, s = OK.quantize_int8(x[n])
        np.testing.assert_array_equal(codes[slot // 16, slot % 16], c)
        np.testing.assert_array_equal(scale[slot // 16, slot % 16], s)
    packed = np.zeros((2, 16, 2, 64), np.uint8)
    sz = np.zeros((2, 16, 2, 4, 2), np.float16)
    OK.append_kv(packed, x, [3, 16, 30], 16, "int4", sz)
    for n, slot in enumerate([3, 16, 30]):
        p, s = OK.quantize_int4(x[n])
        np.testing.assert_array_equal(packed[slot // 16, slot % 16], p)
        np.testing.assert_array_equal(sz[slot // 16, slot % 16], s)
