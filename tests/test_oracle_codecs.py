"""Pins of the oracle's codecs against library routines and the OCP tables (CPU)."""
import math

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from tests import brute


def test_decode_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3(codes)
    ref = brute.e4m3_table()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))  # -0 is 0x80
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and ours[0x7E] == 448.0


def test_decode_e5m2_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e5m2(codes)
    ref = brute.e5m2_table()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])  # includes +-inf at 0x7C / 0xFC
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def test_decode_e5m2_hand_values():
    # OCP FP8 E5M2: bias 15, largest finite 0x7B = 1.75 * 2**15, smallest subnormal 2**-16
    v = O.decode_e5m2(np.array([0x3C, 0x3D, 0x7B, 0x01, 0x03, 0x04, 0x7C, 0xBC, 0x80], np.uint8))
    assert list(v[:6]) == [1.0, 1.25, 57344.0, 2.0 ** -16, 3 * 2.0 ** -16, 2.0 ** -14]
    assert v[6] == np.inf and v[7] == -1.0 and v[8] == 0.0 and np.signbit(v[8])


def test_dequant_weight_e5m2_block_scales():
    rng = np.random.default_rng(4)
    w = (rng.integers(0, 0x7C, (256, 256)) | (rng.integers(0, 2, (256, 256)) << 7)).astype(np.uint8)
    sf = rng.integers(110, 135, (2, 2), dtype=np.uint8)
    ours = O.dequant_weight(w, sf, "fp8e5m2", 256, 256)
    ref = brute.weight_dense(w, sf, "fp8e5m2", 256, 256)
    assert np.array_equal(ours, ref)
    # the same bytes read as E4M3 give different values: the format switch is live
    assert not np.array_equal(ours, O.dequant_weight(w, sf, "fp8", 256, 256))


def _midpoints_and_values():
    vals = np.unique(brute.e4m3_table()[:0x7F])  # non-negative finite values
    mids = (vals[1:] + vals[:-1]) / 2
    # quarter points either side of each midpoint exercise the round-up/down decisions
    q = (vals[1:] - vals[:-1]) / 4
    return np.concatenate([vals, mids, mids - q, mids + q])


def test_encode_e4m3_rne_matches_torch_on_ties_and_grid():
    v = _midpoints_and_values()
    v = np.concatenate([v, -v])
    ours = O.encode_e4m3_rne(v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_e4m3_rne_matches_torch_random():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-448, 448, 200000), rng.normal(0, 0.01, 200000),
                        rng.normal(0, 1e-3, 50000)]).astype(np.float32)
    ours = O.encode_e4m3_rne(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_e4m3_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.encode_e4m3_rne(np.array([449.0]))
    with pytest.raises(ValueError):
        O.encode_e4m3_rne(np.array([np.nan]))


def test_decode_ue8m0_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = O.decode_ue8m0(b)
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


def test_decode_e2m1_matches_ocp_table():
    nib = np.arange(16, dtype=np.uint8)
    ours = O.decode_e2m1(nib)
    ref = np.array([brute.e2m1_value(int(n)) for n in nib])
    assert np.array_equal(ours, ref)


def test_bf16_rne_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(1)
    v = rng.normal(0, 3, 300000).astype(np.float32)
    # exact ties between two bf16 neighbours: low 16 bits = 0x8000
    ties = ((rng.integers(0, 1 << 14, 20000, dtype=np.uint32) + 0x3000) << 16 | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties, np.array([0.0, -0.0], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = O.bf16_rne_bits(v.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_bf16_single_rounding_from_float64():
    # a float64 just above a bf16 midpoint must round up even though its float32 rounding is the midpoint
    mid = 1.0 + 2.0 ** -8  # halfway between 1.0 and 1.0078125
    v = np.array([mid + 2.0 ** -40, mid - 2.0 ** -40, mid])
    bits = O.bf16_rne_bits(v)
    assert list(bits) == [0x3F81, 0x3F80, 0x3F80]


def test_dequant_weight_fp8_block_scales():
    rng = np.random.default_rng(2)
    w = (rng.integers(0, 0x7E, (256, 384)) | (rng.integers(0, 2, (256, 384)) << 7)).astype(np.uint8)
    sf = rng.integers(120, 135, (2, 3), dtype=np.uint8)
    ours = O.dequant_weight(w, sf, "fp8", 256, 384)
    ref = brute.weight_dense(w, sf, "fp8", 256, 384)
    assert np.array_equal(ours, ref)


def test_dequant_weight_mxfp4_nibble_order():
    rng = np.random.default_rng(3)
    w = rng.integers(0, 256, (8, 32), dtype=np.uint8)
    sf = rng.integers(120, 135, (8, 2), dtype=np.uint8)
    ours = O.dequant_weight(w, sf, "mxfp4", 8, 64)
    ref = brute.weight_dense(w, sf, "mxfp4", 8, 64)
    assert np.array_equal(ours, ref)
    # element 0 of a row is the low nibble of byte 0
    one = np.zeros((1, 16), np.uint8)
    one[0, 0] = 0x02  # low nibble 0b0010 = 1.0, high nibble 0
    v = O.dequant_weight(one, np.full((1, 1), 127, np.uint8), "mxfp4", 1, 32)
    assert v[0, 0] == 1.0 and np.all(v[0, 1:] == 0)
