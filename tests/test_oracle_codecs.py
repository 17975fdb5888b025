"""Pins for the oracle's number formats (no GPU).

The codecs are checked against their definitions and against PyTorch's CPU
dtype conversions (library routines), exhaustively where the format is small.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_fp8_points_from_the_format_definition():
    rows = []
    with open(os.path.join(GOLDEN, "fp8_e4m3fn_points.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                code, val = line.split()
                rows.append((int(code, 16), float(val)))
    assert len(rows) >= 15
    got = codecs.fp8_e4m3_to_f64(np.array([c for c, _ in rows], np.uint8))
    for (code, want), g in zip(rows, got):
        if math.isnan(want):
            assert math.isnan(g), hex(code)
        else:
            assert g == want and math.copysign(1, g) == math.copysign(1, want), hex(code)


def test_fp8_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.fp8_e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert np.nanmax(ours) == 448.0 and np.isnan(ours).sum() == 2


def test_bf16_decode_all_65536_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = codecs.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def _bf16_torch(x32):
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_random_and_edges():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2**32, size=1 << 24, dtype=np.uint64).astype(np.uint32)
    edges = np.array([0x00000000, 0x80000000, 0x00000001, 0x807FFFFF, 0x3F808000, 0x3F818000,
                      0x3F80FFFF, 0x3F807FFF, 0x7F7FFFFF, 0x7F7F8000, 0x7F800000, 0xFF800000,
                      0x7FC00000, 0xFFC00001, 0x00008000, 0x00018000, 0x3F7F8000],
                     dtype=np.uint32)
    x = np.concatenate([bits, edges]).view(np.float32)
    ours = codecs.f32_to_bf16_rne(x)
    ref = _bf16_torch(x)
    nan = np.isnan(x)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(np.isnan(codecs.bf16_to_f64(ours[nan])))


def test_bf16_ties_go_to_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: even is 1.0
    x = np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8], np.float32)
    assert list(codecs.bf16_to_f64(codecs.f32_to_bf16_rne(x))) == [1.0, 1.0 + 2 * 2.0**-7]


@pytest.mark.parametrize("scale", [1.0, 0.0087890625, 4.1 / 448.0, 3.0e-3, 1.7])
def test_fp8_dequant_matches_torch_route(scale):
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.fp8_e4m3_dequant_bf16(codes, scale)
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
    ref = (v * torch.tensor(scale, dtype=torch.float32)).to(torch.bfloat16)
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(codecs.fp8_e4m3_to_f64(codes))
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(np.isnan(codecs.bf16_to_f64(ours[nan])))


def test_dequant_rounds_the_product_to_nearest():
    # 1.0 * (1 + 2^-8 + 2^-10) lies above the midpoint between the bf16
    # neighbours 1 and 1 + 2^-7, so rounding (not truncation) gives 1 + 2^-7
    scale = 1.0 + 2.0**-8 + 2.0**-10
    out = codecs.bf16_to_f64(codecs.fp8_e4m3_dequant_bf16(np.array([0x38, 0xB8], np.uint8), scale))
    assert list(out) == [1.0 + 2.0**-7, -(1.0 + 2.0**-7)]
