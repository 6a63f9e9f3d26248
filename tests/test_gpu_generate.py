"""Greedy generation on the device (gpt2_generate) against the oracle's greedy loop.

The oracle side is the plain loop the pages describe: cachedStep at each position,
the next token the first maximum of the logits (numpy argmax), and rejection of
non-finite logits.  The fp32 choices must agree with the oracle's wherever the
oracle's top-2 gap exceeds 1e-2 (past the first step where it does not, the two
sequences may legitimately part); the int8 choices and logits are bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
import stream_gpt_transformer_amd as g
import synth
from gpu_common import ARGMAX_GAP, D, PER, TOL_F32, checkpoint, model, need_gpu, oracle_q8

pytestmark = pytest.mark.gpu


def oracle_greedy(w, prompt, n_gen, q8=None):
    """Returns (chosen tokens, top-2 gap of each choice's logits, last logits)."""
    oracle.set_threads(16)
    n = len(prompt) + n_gen - 1
    cache = np.zeros(n * PER, np.float32)
    toks, gaps, tok, lg = [], [], None, None
    for p in range(n):
        t = int(prompt[p]) if p < len(prompt) else tok
        if q8 is None:
            rc, lg = oracle.cached_step(D, w, cache, p * PER, t, p)
        else:
            rc, lg = oracle.q8_cached_step(D, w, q8[0], q8[1], cache, p * PER, t, p)
        assert rc == 0
        if p >= len(prompt) - 1:
            assert np.all(np.isfinite(lg))
            tok = int(np.argmax(lg))
            top2 = np.sort(lg)[-2:]
            toks.append(tok)
            gaps.append(float(top2[1] - top2[0]))
    return toks, gaps, lg


def gpu_generate(m, prompt, n_gen, q8=False):
    n = len(prompt) + n_gen - 1
    cache = torch.zeros(n * PER, dtype=torch.float32, device="cuda")
    logits = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    out = torch.full((n_gen,), -1, dtype=torch.int32, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    m.generate(cache, prompt, n_gen, logits, out, status, q8=q8)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32).tolist(), int(status.item()), logits.cpu().numpy()


PROMPT = synth.make_tokens(synth.SEED_SHORT, 8).tolist()


def test_generate_fp32_matches_oracle_greedy():
    need_gpu()
    n_gen = 24
    toks, status, lg = gpu_generate(model(), PROMPT, n_gen)
    ref, gaps, ref_lg = oracle_greedy(checkpoint(), PROMPT, n_gen)
    assert status == 0
    for i in range(n_gen):
        if gaps[i] <= ARGMAX_GAP:  # a near tie: the sequences may part here
            break
        assert toks[i] == ref[i], f"choice {i}: {toks[i]} vs oracle {ref[i]} (gap {gaps[i]:.3e})"
    else:
        assert np.abs(lg - ref_lg).max() <= TOL_F32


def test_generate_int8_bit_identical_to_oracle_greedy():
    need_gpu()
    n_gen = 16
    toks, status, lg = gpu_generate(model(), PROMPT, n_gen, q8=True)
    ref, _, ref_lg = oracle_greedy(checkpoint(), PROMPT, n_gen, q8=oracle_q8())
    assert status == 0
    assert toks == ref
    assert np.array_equal(lg.view(np.uint32), ref_lg.view(np.uint32))


def test_generate_per_phase_path_same_choices():
    """The per-phase kernels (the fallback when the single-launch step cannot run)
    read the fed token the same way: same choices and logits as the fused path."""
    need_gpu()
    m = model()
    fused = gpu_generate(m, PROMPT, 12)
    g.gpt2_test_force_phase_kernels(1)
    try:
        phase = gpu_generate(m, PROMPT, 12)
    finally:
        g.gpt2_test_force_phase_kernels(0)
    assert fused[0] == phase[0] and fused[1] == phase[1] == 0
    assert np.array_equal(fused[2].view(np.uint32), phase[2].view(np.uint32))


def test_generate_single_token_prompt_and_full_length():
    """n_prompt = 1 and the longest run (n_prompt + n_gen - 1 = 128 positions)."""
    need_gpu()
    m = model()
    toks, status, _ = gpu_generate(m, PROMPT[:1], 128)
    assert status == 0 and len(toks) == 128 and max(toks) < g.GPT2_VOCAB
    ref, gaps, _ = oracle_greedy(checkpoint(), PROMPT[:1], 4)
    for i in range(4):
        if gaps[i] <= ARGMAX_GAP:
            break
        assert toks[i] == ref[i]


def test_generate_rejects_nonfinite_logits():
    """A final-LayerNorm gain of NaN makes every logit NaN: the first choice is
    rejected (status 1) and every choice is 50,257."""
    need_gpu()
    w = checkpoint().copy()
    o, _ = synth.offsets(D)["lnf_g"]
    w[o] = np.nan
    m = g.Model(torch.from_numpy(w).cuda(), g.GPT2_PACK_F32)
    toks, status, lg = gpu_generate(m, PROMPT[:4], 5)
    assert status == 1
    assert toks == [g.GPT2_VOCAB] * 5
    m.close()


def test_generate_validation():
    need_gpu()
    m = model()
    cap = 40 * PER
    cache = torch.zeros(cap, dtype=torch.float32, device="cuda")
    lg = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    out = torch.empty(64, dtype=torch.int32, device="cuda")
    st = torch.empty(1, dtype=torch.int32, device="cuda")

    def call(prompt=(1, 2, 3), n_gen=4, weights=0, cap_words=cap, cache_p=None, out_p=None):
        return g.gpt2_generate(m.handle, cache.data_ptr() if cache_p is None else cache_p, cap_words, list(prompt),
                               n_gen, weights, m.ws.data_ptr(), lg.data_ptr(),
                               out.data_ptr() if out_p is None else out_p, st.data_ptr())

    assert call(prompt=()) == g.GPT2_ETOKEN
    assert call(n_gen=0) == g.GPT2_ETOKEN
    assert call(prompt=[1] * 100, n_gen=30) == g.GPT2_ETOKEN       # 129 positions
    assert call(prompt=[1, g.GPT2_VOCAB]) == g.GPT2_ETOKEN
    assert call(cap_words=5 * PER) == g.GPT2_ECACHE                 # needs 6 positions
    assert call(cache_p=0) == g.GPT2_ECACHE
    assert call(out_p=0) == g.GPT2_EARG
    assert call(weights=3) == g.GPT2_EARG
    assert call(weights=-1) == g.GPT2_EARG
    assert call(weights=g.GPT2_WEIGHTS_F16) == g.GPT2_ENOTPACKED     # packed fp32 + int8 only
    torch.cuda.synchronize()
    mf = model(flags=g.GPT2_PACK_F32)
    assert g.gpt2_generate(mf.handle, cache.data_ptr(), cap, [1], 2, 1, mf.ws.data_ptr(), lg.data_ptr(),
                           out.data_ptr(), st.data_ptr()) == g.GPT2_ENOTPACKED
