"""The GPU's exponential and tanh against the oracle's, bit for bit, over every one
of the 2^32 binary32 bit patterns (the muInference page checks its exponential by
enumerating all 2^32 inputs)."""
import numpy as np
import pytest
import torch

import oracle
import stream_gpt_transformer_amd as g
from gpu_common import need_gpu

pytestmark = pytest.mark.gpu

CHUNK = 1 << 26


@pytest.mark.parametrize("kind", [0, 1], ids=["exp", "tanh"])
def test_all_bit_patterns_match_oracle(kind):
    need_gpu()
    oracle.set_threads(16)
    y = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    mismatches = 0
    for c in range((1 << 32) // CHUNK):
        first = c * CHUNK
        assert g.gpt2_test_special(kind, first, CHUNK, y.data_ptr(), 0) == 0
        ref = oracle.special_bits(kind, first, CHUNK)
        got = y.cpu().numpy()
        diff = got.view(np.uint32) != ref.view(np.uint32)
        if diff.any():
            both_nan = np.isnan(got) & np.isnan(ref)
            mismatches += int((diff & ~both_nan).sum())
    assert mismatches == 0
