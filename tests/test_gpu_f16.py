"""The cached step with binary16 weight storage (gpt2.s page, options, -h) on the GPU.

- 128-position session against the oracle's binary16 step (oracle_f16_cached_step):
  max |logit difference| <= 2e-3, greedy agreement where the oracle's top-2 gap
  exceeds 1e-2, caches within 1e-4 (the arithmetic is the fp32 step's).
- Bit identity with the GPU fp32 step on a checkpoint whose block matrices and
  token table hold numpy-rounded binary16 values, for tokens whose embedding rows
  are binary16 values already (the binary16 step reads the embedding from the
  binary32 table): same logits and caches to the bit over 40 positions, with random
  biases and LayerNorm parameters.
- The single-launch kernel against the per-phase kernels (same bits), greedy
  generation against a host loop of binary16 steps, and the rejections.
"""
import numpy as np
import pytest
import torch

import stream_gpt_transformer_amd as g
import synth
from gpu_common import (D, PER, TOL_F32, check_logits, checkpoint, gpu_session, model, need_gpu,
                        oracle_session_f16)

pytestmark = pytest.mark.gpu


def test_f16_session_matches_oracle():
    need_gpu()
    toks = synth.make_tokens(synth.SEED_SESSION, 128)
    ref, ref_cache = oracle_session_f16(0, tuple(toks.tolist()))
    got, cache = gpu_session(model(flags=g.GPT2_PACK_F16), toks, f16=True)
    check_logits(got, ref, TOL_F32, "binary16 128-step session")
    assert np.abs(cache - ref_cache).max() <= 1e-4


def _half(v):
    return v.astype(np.float16).astype(np.float32)


def test_f16_step_equals_fp32_step_on_rounded_checkpoint():
    need_gpu()
    toks = synth.make_tokens(33, 40)
    w = checkpoint(1, True).copy()
    off = synth.offsets(D)
    o, n = off["wte"]
    wte = w[o:o + n].reshape(g.GPT2_VOCAB, g.GPT2_DMODEL)
    wte[np.unique(toks)] = _half(wte[np.unique(toks)])  # these rows: binary16 values already
    wr = w.copy()
    for name, (o, n) in off.items():
        if name == "wte" or name.endswith("_w"):
            wr[o:o + n] = _half(w[o:o + n])
    m16 = g.Model(torch.from_numpy(w).cuda(), g.GPT2_PACK_F16)
    m32 = g.Model(torch.from_numpy(wr).cuda(), g.GPT2_PACK_F32)
    torch.cuda.synchronize()
    try:
        a, ca = gpu_session(m16, toks, f16=True)
        b, cb = gpu_session(m32, toks)
    finally:
        m16.close()
        m32.close()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(ca.view(np.uint32), cb.view(np.uint32))


def test_f16_fused_step_equals_phase_kernels():
    need_gpu()
    m = model(flags=g.GPT2_PACK_F32 | g.GPT2_PACK_F16)
    toks = synth.make_tokens(21, 40)
    fused, cf = gpu_session(m, toks, f16=True)
    g.gpt2_test_force_phase_kernels(True)
    try:
        phase, cp = gpu_session(m, toks, f16=True)
    finally:
        g.gpt2_test_force_phase_kernels(False)
    assert np.array_equal(fused.view(np.uint32), phase.view(np.uint32))
    assert np.array_equal(cf.view(np.uint32), cp.view(np.uint32))
    # and it is not the fp32 step
    f32, _ = gpu_session(m, toks)
    assert not np.array_equal(fused, f32)


def test_f16_generate_equals_host_loop():
    """gpt2_generate with binary16 weights chooses the first maximum of each step's
    logits: the same tokens as a host loop of gpt2_f16_cached_step calls, and the
    same last logits to the bit."""
    need_gpu()
    m = model(flags=g.GPT2_PACK_F16)
    prompt = synth.make_tokens(44, 6).tolist()
    n_gen = 30
    n = len(prompt) + n_gen - 1
    cache = torch.zeros(n * PER, dtype=torch.float32, device="cuda")
    lg = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    out = torch.empty(n_gen, dtype=torch.int32, device="cuda")
    st = torch.empty(1, dtype=torch.int32, device="cuda")
    m.generate(cache, prompt, n_gen, lg, out, st, f16=True)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = out.cpu().numpy().tolist()

    hc = m.new_cache(n)
    hl = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    want, tok = [], None
    for p in range(n):
        m.step(hc, p, prompt[p] if p < len(prompt) else tok, hl, f16=True)
        if p >= len(prompt) - 1:
            tok = int(torch.argmax(hl).item())  # torch returns the first maximum
            want.append(tok)
    torch.cuda.synchronize()
    assert got == want
    assert np.array_equal(lg.cpu().numpy().view(np.uint32), hl.cpu().numpy().view(np.uint32))
    assert torch.equal(cache, hc)


def test_f16_rejections():
    need_gpu()
    mf = model(flags=g.GPT2_PACK_F32)
    cache = mf.new_cache(2)
    lg = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    assert g.gpt2_f16_cached_step(mf.handle, cache.data_ptr(), 0, 1, 0, mf.ws.data_ptr(),
                                  lg.data_ptr()) == g.GPT2_ENOTPACKED
    m = model(flags=g.GPT2_PACK_F16)
    ws, lp = m.ws.data_ptr(), lg.data_ptr()
    assert g.gpt2_f16_cached_step(m.handle, cache.data_ptr(), 0, g.GPT2_VOCAB, 0, ws, lp) == g.GPT2_ETOKEN
    assert g.gpt2_f16_cached_step(m.handle, cache.data_ptr(), PER, 1, 0, ws, lp) == g.GPT2_ECACHE
    assert g.gpt2_f16_cached_step(m.handle, cache.data_ptr(), 0, 1, 128, ws, lp) == g.GPT2_EPOSITION
    # the fp32 and int8 steps need their own packed forms
    assert g.gpt2_cached_step(m.handle, cache.data_ptr(), 0, 1, 0, ws, lp) == g.GPT2_ENOTPACKED
    assert g.gpt2_q8_cached_step(m.handle, cache.data_ptr(), 0, 1, 0, ws, lp) == g.GPT2_ENOTPACKED
