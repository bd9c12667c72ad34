"""The oracle decodes fp16/bf16 bit patterns itself; check every one of the 65536 patterns
against torch's own conversion of the same bits to float64."""
import numpy as np
import pytest
import torch

import oracle


@pytest.mark.parametrize("dtype,code", [(torch.float16, oracle.F16), (torch.bfloat16, oracle.BF16)])
def test_decode_exhaustive(dtype, code):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.decode_array(bits, code)
    ref = torch.from_numpy(bits.view(np.int16)).view(dtype).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))
