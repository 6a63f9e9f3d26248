"""gpt2_cached_step_noalloc (the batch-1 fp32 step on the library's own static
scratch, for callers that cannot allocate) against gpt2_cached_step on the same
inputs: logits and the appended cache rows bit for bit, on two calls in a row, the
second with a smaller input (fewer cached positions)."""
import numpy as np
import pytest
import torch

import stream_gpt_transformer_amd as g
import synth
from gpu_common import model, need_gpu

PER = g.GPT2_CACHE_WORDS_PER_POS


def _prefix_cache(m, toks, n):
    """A cache holding positions 0..n-1 of the session (room for one more)."""
    cache = m.new_cache(n + 1)
    lg = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    for p in range(n):
        m.step(cache, p, int(toks[p]), lg)
    return cache


@pytest.mark.gpu
def test_noalloc_step_equals_cached_step_twice_shrinking():
    need_gpu()
    m = model(0)
    toks = synth.make_tokens(synth.SEED_SHORT, 8)
    s = torch.cuda.current_stream().cuda_stream
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    for pos in (6, 2):  # the second call has the smaller input
        base = _prefix_cache(m, toks, pos)
        c_ref, c_na = base.clone(), base.clone()
        l_ref = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
        l_na = torch.full((g.GPT2_VOCAB,), float("nan"), dtype=torch.float32, device="cuda")
        rc = g.gpt2_cached_step(m.handle, c_ref.data_ptr(), pos * PER, int(toks[pos]), pos, m.ws.data_ptr(),
                                l_ref.data_ptr(), s)
        assert rc == g.GPT2_OK
        status.fill_(-1)
        rc = g.gpt2_cached_step_noalloc(m.handle, c_na.data_ptr(), pos * PER, int(toks[pos]), pos, l_na.data_ptr(),
                                        status.data_ptr(), s)
        assert rc == g.GPT2_OK
        torch.cuda.synchronize()
        print(f"noalloc position {pos}: status {int(status.item())}", flush=True)
        assert int(status.item()) == 0
        assert m.status() == 0
        assert torch.equal(l_na.view(torch.int32), l_ref.view(torch.int32)), f"logits differ at position {pos}"
        assert torch.equal(c_na.view(torch.int32), c_ref.view(torch.int32)), f"cache differs at position {pos}"
    # a status pointer is optional
    pos = 1
    base = _prefix_cache(m, toks, pos)
    l_na = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    assert g.gpt2_cached_step_noalloc(m.handle, base.data_ptr(), pos * PER, int(toks[pos]), pos, l_na.data_ptr(),
                                      None, s) == g.GPT2_OK
    torch.cuda.synchronize()
    assert np.isfinite(l_na.cpu().numpy()).all()


@pytest.mark.gpu
def test_noalloc_step_rejects_bad_arguments_before_enqueuing():
    need_gpu()
    m = model(0)
    lg = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    cache = m.new_cache(2)
    c, l = cache.data_ptr(), lg.data_ptr()
    assert g.gpt2_cached_step_noalloc(m.handle, c, 0, g.GPT2_VOCAB, 0, l) == g.GPT2_ETOKEN
    assert g.gpt2_cached_step_noalloc(m.handle, c, 0, 0, 128, l) == g.GPT2_EPOSITION
    assert g.gpt2_cached_step_noalloc(m.handle, c, PER, 0, 0, l) == g.GPT2_ECACHE
    assert g.gpt2_cached_step_noalloc(m.handle, c, 0, 0, 0, 0) == g.GPT2_EARG
    assert g.gpt2_cached_step_noalloc(m.handle, c, 0, 0, 0, l, l + 2) == g.GPT2_EARG
