"""The kernels' fp8 E4M3FN -> bf16 dequant, bit for bit against the oracle's
codec over all 256 codes and several per-tensor scales [DCP-PR, 3.2 figure:
fp8 cache rows are converted to bf16 and scaled; OCP 8-bit FP, E4M3]."""
import numpy as np
import pytest
import torch

from oracle import codecs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("scale", [1.0, 0.0087890625, 4.1 / 448.0, 3.0e-3, 1.7, 2.0**-10])
def test_all_codes_bit_exact(gpu, scale):
    codes = np.tile(np.arange(256, dtype=np.uint8), 5)[:1021]  # ragged tail
    out = gpu.fp8_dequant_bf16(torch.from_numpy(codes).cuda(), scale)
    got = out.cpu().numpy().view(np.uint16)
    want = codecs.fp8_e4m3_dequant_bf16(codes, scale)
    nan = np.isnan(codecs.fp8_e4m3_to_f64(codes))
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all(np.isnan(codecs.bf16_to_f64(got[nan])))
