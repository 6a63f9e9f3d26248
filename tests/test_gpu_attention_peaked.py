"""Attention outside the near-uniform regime (LeanExe GPT-2 README, cachedStep
paragraph: causal attention over the cached keys and values).

The seed-0 weights give scores of about N(0, 0.3^2), so softmax weights are close
to uniform.  The "peaked" checkpoint (synth.make_checkpoint(..., peaked=True))
scales every block's query and key columns by 10: scores spread over tens of units,
most exp arguments fall below -87 (where the specified exponential returns 0) and
the weights are close to one-hot.  Position rows 5, 9 and 17 are equal and the
session repeats one token there, so layer 0 has tied keys.

- The workload really is in that regime: the oracle's own layer-0 attention at the
  last position has weights that are exactly 0 and a largest weight above 0.9.
- fp32 single-launch step.  This regime is ill-conditioned in binary32: the oracle's
  own logits are up to 4.0e-3 from transformers' GPT-2 in float64 (5e-6 on the
  plain checkpoint), so any other summation order lands about as far from it, and
  the 2e-3 bound against the oracle cannot hold at every position.  The test takes
  the float64 model as the yardstick: the GPU's largest logit error against it is
  at most twice the oracle's; at positions where the oracle is within 1e-3 of
  float64 the GPU is within 2e-3 of the oracle; greedy choices agree with the
  oracle's wherever its top-2 gap exceeds 1e-2; the cache's largest error against
  the float64 keys and values is at most twice the oracle's.
- int8 single-launch step and int8 per-phase kernels: logits and cache bit-identical
  to the oracle's int8 session.
- Batched step: four sessions of this checkpoint advanced together equal their
  batch-1 runs bit for bit.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import stream_gpt_transformer_amd as g
import synth
from gpu_common import D, PER, TOL_F32, check_logits, checkpoint, gpu_session, model, need_gpu

pytestmark = pytest.mark.gpu

T = 40  # positions 0..39 (past every tied position)


@functools.lru_cache(maxsize=None)
def _tokens():
    return synth.make_tied_tokens(synth.SEED_PEAKED, T)


@functools.lru_cache(maxsize=None)
def _oracle(q8: bool):
    w = checkpoint(0, False, True)
    oracle.set_threads(16)
    return oracle.session(D, w, _tokens(), q8=oracle.q8_quantize_weights(D, w) if q8 else None)


def _model():
    return model(0, False, 3, True)


def test_workload_is_peaked_with_underflow_and_ties():
    """Layer-0 attention of head 0 at the last position, by the oracle's own functions
    (layer-0 keys and values from its session cache)."""
    need_gpu()
    w = checkpoint(0, False, True)
    off = synth.offsets(D)
    toks = _tokens()
    _, cache = _oracle(False)
    p = T - 1
    wte = w[off["wte"][0]:off["wte"][0] + off["wte"][1]].reshape(-1, 768)
    wpe = w[off["wpe"][0]:off["wpe"][0] + off["wpe"][1]].reshape(-1, 768)
    x = (wte[int(toks[p])] + wpe[p]).astype(np.float32)  # the embedding sum, one fp32 add per element
    blk = lambda name: w[off[f"h0.{name}"][0]:off[f"h0.{name}"][0] + off[f"h0.{name}"][1]]
    xn = oracle.layernorm(x, blk("ln1_g"), blk("ln1_b"))
    q = oracle.linear(xn, blk("attn_w").reshape(768, 2304)[:, :64].copy(), blk("attn_b")[:64].copy())
    rows = cache[:T * PER].reshape(T, 12, 1536)[:, 0, :]
    K, V = rows[:, 0:64].copy(), rows[:, 768:832].copy()
    assert np.array_equal(K[synth.PEAK_TIED_POSITIONS[0]], K[synth.PEAK_TIED_POSITIONS[1]])
    _, wts = oracle.attention_head(q, K, V)
    assert (wts == 0.0).sum() >= 5, wts
    assert wts.max() > 0.9, wts.max()


@functools.lru_cache(maxsize=None)
def _float64():
    import hf_ref
    m = hf_ref.build(checkpoint(0, False, True), D)
    return hf_ref.logits_all_positions(m, _tokens()), hf_ref.cache_all_positions(m, _tokens(), D)


def test_peaked_fp32_session_against_oracle_and_float64():
    need_gpu()
    ref, ref_cache = _oracle(False)
    got, cache = gpu_session(_model(), _tokens())
    exact, exact_cache = _float64()
    e_or = np.abs(ref.astype(np.float64) - exact).max(axis=1)
    e_gpu = np.abs(got.astype(np.float64) - exact).max(axis=1)
    print(f"peaked fp32: max |oracle - float64| {e_or.max():.3e}, max |gpu - float64| {e_gpu.max():.3e}, "
          f"max |gpu - oracle| {np.abs(got - ref).max():.3e}", flush=True)
    assert e_gpu.max() <= 2.0 * e_or.max()
    calm = e_or <= 1e-3
    assert calm.sum() >= 10
    check_logits(got[calm], ref[calm], TOL_F32, "peaked fp32 session, well-conditioned positions")
    check_logits(got, ref, np.inf, "peaked fp32 session, greedy agreement")
    c_or = np.abs(ref_cache.astype(np.float64) - exact_cache).max()
    c_gpu = np.abs(cache[:T * PER].astype(np.float64) - exact_cache).max()
    print(f"peaked fp32 cache: max |oracle - float64| {c_or:.3e}, max |gpu - float64| {c_gpu:.3e}", flush=True)
    assert c_gpu <= 2.0 * c_or


@pytest.mark.parametrize("phase_kernels", [False, True])
def test_peaked_int8_session_bit_identical(phase_kernels):
    need_gpu()
    ref, ref_cache = _oracle(True)
    g.gpt2_test_force_phase_kernels(phase_kernels)
    try:
        got, cache = gpu_session(_model(), _tokens(), q8=True)
    finally:
        g.gpt2_test_force_phase_kernels(False)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
        f"max |diff| {np.abs(got - ref).max():.3e}"
    assert np.array_equal(cache[:T * PER].view(np.uint32), ref_cache.view(np.uint32))


def test_peaked_batched_equals_batch1():
    need_gpu()
    m = _model()
    B, TB = 4, 24
    toks = np.stack([synth.make_tied_tokens(synth.SEED_PEAKED + 10 + b, TB) for b in range(B)])
    caches = m.new_cache(TB, batch=B)
    out = torch.empty((TB, B, g.GPT2_VOCAB), dtype=torch.float32, device="cuda")
    for p in range(TB):
        rc = g.gpt2_batched_cached_step(m.handle, caches.data_ptr(), caches.shape[1], [p * PER] * B,
                                        toks[:, p].tolist(), [p] * B, m.ws.data_ptr(), out[p].data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
        assert rc == 0
    torch.cuda.synchronize()
    for b in range(B):
        one, one_cache = gpu_session(m, toks[b])
        assert np.array_equal(out[:, b].cpu().numpy().view(np.uint32), one.view(np.uint32)), b
        assert np.array_equal(caches[b].cpu().numpy().view(np.uint32), one_cache.view(np.uint32)), b
