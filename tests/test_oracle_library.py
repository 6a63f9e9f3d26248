"""The oracle against independent library routines in float64.

GPT-2 as a whole: transformers' GPT2LMHeadModel (float64) loaded from the same
packed checkpoint (tests/hf_ref.py).  A transposed matrix, a wrong offset, a
dropped bias or a sign error moves logits by far more than float32 rounding.
Single operations: torch's layer_norm, tanh-GELU and scaled-dot-product attention
and a float64 matrix product.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import hf_ref
import oracle
import synth


def test_tiny_robust_session_matches_transformers(ckpt_tiny_robust):
    d = synth.TINY
    toks = synth.make_tokens(5, d.max_pos, d)
    lg, _ = oracle.session(d, ckpt_tiny_robust, toks)
    ref = hf_ref.logits_all_positions(hf_ref.build(ckpt_tiny_robust, d), toks)
    assert np.abs(ref - lg).max() <= 2e-6 * max(1.0, np.abs(ref).max())


@pytest.mark.slow
def test_tiny_robust_cache_matches_transformers_keys_values(ckpt_tiny_robust):
    """The cache rows (position*layers + layer)*2D + offset hold the float64 library's
    keys and values of that position and layer, within float32 rounding."""
    d = synth.TINY
    toks = synth.make_tokens(7, d.max_pos, d)
    _, cache = oracle.session(d, ckpt_tiny_robust, toks)
    ref = hf_ref.cache_all_positions(hf_ref.build(ckpt_tiny_robust, d), toks, d)
    assert np.abs(cache.astype(np.float64) - ref).max() <= 1e-5


def test_gpt2_seed0_eight_steps_match_transformers(ckpt_gpt2):
    d = synth.GPT2
    toks = synth.make_tokens(synth.SEED_SHORT, 8, d)
    lg, _ = oracle.session(d, ckpt_gpt2, toks)
    ref = hf_ref.logits_all_positions(hf_ref.build(ckpt_gpt2, d), toks)
    # float32 accumulation over 768/3072-term sums through 12 blocks: ~1e-5 here.
    assert np.abs(ref - lg).max() <= 5e-5


def test_layernorm_matches_torch():
    rng = np.random.default_rng(0)
    for n in (64, 768):
        x = (rng.standard_normal(n) * 3 + 1).astype(np.float32)
        g = (1 + 0.1 * rng.standard_normal(n)).astype(np.float32)
        b = (0.1 * rng.standard_normal(n)).astype(np.float32)
        ref = F.layer_norm(torch.from_numpy(x).double(), (n,), torch.from_numpy(g).double(),
                           torch.from_numpy(b).double(), eps=1e-5).numpy()
        assert np.abs(oracle.layernorm(x, g, b) - ref).max() <= 1e-5


def test_gelu_matches_torch_tanh_form():
    x = np.linspace(-8, 8, 4001).astype(np.float32)
    ref = F.gelu(torch.from_numpy(x).double(), approximate="tanh").numpy()
    got = oracle.gelu(x)
    assert np.abs(got - ref).max() <= 4e-6 * max(1, np.abs(ref).max())


def test_linear_matches_float64_product():
    rng = np.random.default_rng(1)
    for K, N in ((64, 192), (768, 300), (3072, 768)):
        x = rng.standard_normal(K).astype(np.float32)
        W = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
        b = (0.1 * rng.standard_normal(N)).astype(np.float32)
        ref = x.astype(np.float64) @ W.astype(np.float64) + b
        got = oracle.linear(x, W, b)
        # sequential float32 sum: |error| <= (K+1) u sum_k |x_k W_kj| + u |b_j|
        bound = (K + 1) * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(W) + np.abs(b))
        assert np.all(np.abs(got - ref) <= bound)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(2)
    for npos in (1, 2, 64, 128):
        q = rng.standard_normal(64).astype(np.float32)
        K = rng.standard_normal((npos, 64)).astype(np.float32)
        V = rng.standard_normal((npos, 64)).astype(np.float32)
        a, wts = oracle.attention_head(q, K, V)
        tq, tk, tv = (torch.from_numpy(t).double() for t in (q[None, None, None, :], K[None, None],
                                                            V[None, None]))
        ref = F.scaled_dot_product_attention(tq, tk, tv).numpy().reshape(64)
        assert np.abs(a - ref).max() <= 1e-5
        sm = torch.softmax(torch.from_numpy(K).double() @ torch.from_numpy(q).double() / 8.0, 0)
        assert np.abs(wts - sm.numpy()).max() <= 1e-6
