"""int8 quantizer granularity variants on the GPU (marXiv 2609.00018 abstract) against
the oracle's variant step.

Weights packed with gpt2_pack_weights_grouped(gw), steps by
gpt2_q8_cached_step_grouped(gx); the oracle's oracle_qv_cached_step on the same
checkpoint and tokens.  As on the group-64 path, every order that decides a code
is the oracle's, so logits and caches must be bit-identical over the session.
Input groups of 64 run in the single-launch kernel (whatever gw is), others in
the per-phase kernels; both are covered.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
import stream_gpt_transformer_amd as g
import synth
from gpu_common import D, PER, checkpoint, gpu_session, need_gpu

pytestmark = pytest.mark.gpu

VARIANTS = [(0, 64), (64, 0), (0, 0), (192, 128), (256, 768), (384, 384), (128, 64)]


@functools.lru_cache(maxsize=None)
def grouped_model(gw: int, seed: int = 0, robust: bool = False) -> g.Model:
    ck = torch.from_numpy(checkpoint(seed, robust)).cuda()
    m = g.Model(ck, g.GPT2_PACK_Q8, q8_weight_group=gw)
    torch.cuda.synchronize()
    del ck
    return m


@functools.lru_cache(maxsize=None)
def oracle_weights(gw: int, seed: int = 0, robust: bool = False):
    return oracle.qv_quantize_weights(D, checkpoint(seed, robust), gw)


def variant_session(m, toks, gx):
    T = len(toks)
    cache = m.new_cache(T)
    out = torch.empty((T, g.GPT2_VOCAB), dtype=torch.float32, device="cuda")
    for p in range(T):
        m.step(cache, p, int(toks[p]), out[p], q8=True, input_group=gx)
    torch.cuda.synchronize()
    assert m.status() == 0
    return out.cpu().numpy(), cache.cpu().numpy()


@pytest.mark.parametrize("gw,gx", VARIANTS, ids=[f"w{a}-x{b}" for a, b in VARIANTS])
def test_variant_session_bit_identical_to_oracle(gw, gx):
    need_gpu()
    toks = synth.make_tokens(55, 12)
    oracle.set_threads(16)
    ref, ref_cache = oracle.qv_session(D, checkpoint(0), toks, gw, gx, oracle_weights(gw))
    got, cache = variant_session(grouped_model(gw), toks, gx)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), np.abs(got - ref).max()
    assert np.array_equal(cache.view(np.uint32), ref_cache.view(np.uint32))


def test_row_scales_robust_weights():
    """Random biases and LayerNorm parameters, one scale per row for weights and inputs."""
    need_gpu()
    toks = synth.make_tokens(56, 10)
    ref, _ = oracle.qv_session(D, checkpoint(1, True), toks, 0, 0, oracle_weights(0, 1, True))
    got, _ = variant_session(grouped_model(0, 1, True), toks, 0)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), np.abs(got - ref).max()


def test_row_weight_scales_fused_equals_phase_kernels():
    """Per-row weight scales with 64-coordinate input groups run in the single-launch
    kernel; the per-phase kernels give the same bits."""
    need_gpu()
    m = grouped_model(0)
    toks = synth.make_tokens(57, 24)
    fused, cf = gpu_session(m, toks, q8=True)
    g.gpt2_test_force_phase_kernels(True)
    try:
        phase, cp = gpu_session(m, toks, q8=True)
    finally:
        g.gpt2_test_force_phase_kernels(False)
    assert np.array_equal(fused.view(np.uint32), phase.view(np.uint32))
    assert np.array_equal(cf.view(np.uint32), cp.view(np.uint32))


def test_grouped_validation():
    need_gpu()
    m = grouped_model(0)
    assert g.gpt2_q8_weight_group(m.handle) == 0
    assert g.gpt2_q8_weight_group(grouped_model(192).handle) == 192
    assert g.gpt2_q8_weight_group(None) == -1
    cache = m.new_cache(1)
    lg = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    for bad in (32, 100, 320, 1536, -64, 3072):
        assert g.gpt2_q8_cached_step_grouped(m.handle, bad, cache.data_ptr(), 0, 1, 0, m.ws.data_ptr(),
                                             lg.data_ptr()) == g.GPT2_EARG
    ck = torch.from_numpy(checkpoint(0)).cuda()
    n = g.gpt2_packed_nbytes(g.GPT2_PACK_Q8)
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    for bad in (32, 1536, -1):
        rc, h = g.gpt2_pack_weights_grouped(ck.data_ptr(), ck.numel() * 4, buf.data_ptr(), n, g.GPT2_PACK_Q8, bad)
        assert rc == g.GPT2_EARG and h is None
    mf = g.Model(ck, g.GPT2_PACK_F32)
    torch.cuda.synchronize()
    assert g.gpt2_q8_cached_step_grouped(mf.handle, 0, cache.data_ptr(), 0, 1, 0, mf.ws.data_ptr(),
                                         lg.data_ptr()) == g.GPT2_ENOTPACKED
    mf.close()
