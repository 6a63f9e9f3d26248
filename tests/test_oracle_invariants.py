"""Invariants the pages fix for the binary32 path, checked on the oracle.

- LeanExe GPT-2 README, cachedStep and verification paragraphs: a session starts
  from an empty cache at position 0 and passes each returned cache on; cached and
  full-prefix execution are compared.  The oracle's infer runs layer-major without
  a cache, so bit equality with the cached chain pins the cache index
  (source*12 + layer)*1536 + offset and the recurrence.
- Attention over a single key returns that key's value row exactly; softmax
  weights are nonnegative and sum to 1 within rounding.
- Invalid weight length, token, position or cache length is rejected (README:
  "returns two empty byte arrays"), leaving outputs untouched.
"""
import numpy as np
import pytest

import oracle
import synth


def test_infer_equals_cached_chain_tiny_every_prefix(ckpt_tiny_robust):
    d = synth.TINY
    toks = synth.make_tokens(7, d.max_pos, d)
    lg, _ = oracle.session(d, ckpt_tiny_robust, toks)
    for t in range(d.max_pos):
        rc, li = oracle.infer(d, ckpt_tiny_robust, toks[:t + 1])
        assert rc == 0
        assert np.array_equal(li, lg[t]), t


def test_infer_equals_cached_chain_gpt2(ckpt_gpt2):
    d = synth.GPT2
    toks = synth.make_tokens(synth.SEED_SHORT, 8, d)
    lg, _ = oracle.session(d, ckpt_gpt2, toks)
    for t in (0, 3, 7):
        rc, li = oracle.infer(d, ckpt_gpt2, toks[:t + 1])
        assert rc == 0
        assert np.array_equal(li, lg[t]), t


def test_cache_rows_hold_layer0_keys_values(ckpt_tiny_robust):
    """Cache word (p*L + 0)*2D + i is key i of layer 0 at position p; +D is value i."""
    d = synth.TINY
    w = ckpt_tiny_robust
    D = d.d_model
    off = synth.offsets(d)
    toks = synth.make_tokens(11, 5, d)
    _, cache = oracle.session(d, w, toks)

    def t(name, shape):
        o, n = off[name]
        return w[o:o + n].reshape(shape)

    for p in range(5):
        x = (t("wte", (d.vocab, D))[toks[p]] + t("wpe", (d.n_pos_rows, D))[p]).astype(np.float32)
        h = oracle.layernorm(x, t("h0.ln1_g", (D,)).copy(), t("h0.ln1_b", (D,)).copy())
        qkv = oracle.linear(h, t("h0.attn_w", (D, 3 * D)).copy(), t("h0.attn_b", (3 * D,)).copy())
        base = (p * d.n_layer + 0) * 2 * D
        assert np.array_equal(cache[base:base + D], qkv[D:2 * D])
        assert np.array_equal(cache[base + D:base + 2 * D], qkv[2 * D:])


def test_single_key_attention_returns_value_exactly():
    rng = np.random.default_rng(1)
    for dh in (16, 64):
        q = rng.standard_normal(dh).astype(np.float32)
        K = rng.standard_normal((1, dh)).astype(np.float32)
        V = rng.standard_normal((1, dh)).astype(np.float32)
        a, wts = oracle.attention_head(q, K, V)
        assert wts[0] == 1.0
        assert np.array_equal(a, V[0])


def test_dominant_key_with_underflowing_rest_returns_its_value_exactly():
    """Peaked scores: when every other score lies more than 87 below the largest, the
    specified exponential returns exactly 0 for them, so Z = 1, the weights are one-hot
    and the output is the dominant key's value row, bit for bit, wherever it sits."""
    rng = np.random.default_rng(3)
    for npos, top in ((2, 0), (17, 9), (128, 127), (100, 37)):
        q = np.zeros(64, np.float32)
        q[0] = 8.0
        K = rng.standard_normal((npos, 64)).astype(np.float32)
        K[:, 0] = -100.0 + rng.random(npos).astype(np.float32)  # scores (q.k)*0.125 near -100
        K[top, 0] = 20.0                                        # score 20
        V = rng.standard_normal((npos, 64)).astype(np.float32)
        a, wts = oracle.attention_head(q, K, V)
        expect = np.zeros(npos, np.float32)
        expect[top] = 1.0
        assert np.array_equal(wts, expect), (npos, top)
        assert np.array_equal(a, V[top]), (npos, top)


def test_tied_top_keys_share_the_weight():
    """Two equal keys with the largest score: equal weights, each within rounding of 1/2
    when the rest underflow."""
    rng = np.random.default_rng(4)
    q = np.zeros(64, np.float32)
    q[0] = 8.0
    K = rng.standard_normal((40, 64)).astype(np.float32)
    K[:, 0] = -100.0
    K[5, 0] = K[17, 0] = 20.0
    K[17] = K[5]
    V = rng.standard_normal((40, 64)).astype(np.float32)
    a, wts = oracle.attention_head(q, K, V)
    assert wts[5] == wts[17] == np.float32(0.5)
    assert np.count_nonzero(wts) == 2
    assert np.array_equal(a, (np.float32(0.5) * V[5]) + np.float32(0.5) * V[17])


def test_softmax_mass_and_order():
    rng = np.random.default_rng(2)
    for npos in (2, 17, 128):
        q = rng.standard_normal(64).astype(np.float32)
        K = rng.standard_normal((npos, 64)).astype(np.float32)
        V = rng.standard_normal((npos, 64)).astype(np.float32)
        _, wts = oracle.attention_head(q, K, V)
        assert np.all(wts >= 0)
        assert abs(float(np.sum(wts, dtype=np.float64)) - 1.0) <= npos * 2.0 ** -23
        scores = K.astype(np.float64) @ q.astype(np.float64)
        assert int(np.argmax(wts)) == int(np.argmax(scores))


def test_thread_count_does_not_change_bits(ckpt_tiny_robust):
    d = synth.TINY
    toks = synth.make_tokens(3, 6, d)
    oracle.set_threads(1)
    a, ca = oracle.session(d, ckpt_tiny_robust, toks)
    oracle.set_threads(8)
    b, cb = oracle.session(d, ckpt_tiny_robust, toks)
    assert np.array_equal(a, b) and np.array_equal(ca, cb)


def test_validation_rejects_and_leaves_outputs(ckpt_tiny_robust):
    d = synth.TINY
    w = ckpt_tiny_robust
    per = oracle.cache_words_per_pos(d)
    cache = np.zeros(3 * per, np.float32)
    lib = oracle.lib()
    dd = oracle.dims(d)
    import ctypes

    def step(wt, cw, tok, pos):
        lg = np.full(d.vocab, 7.0, np.float32)
        c = cache.copy()
        rc = lib.oracle_cached_step(ctypes.byref(dd), wt, wt.size, c, cw, tok, pos, lg)
        return rc, lg, c

    cases = [
        (w[:-1].copy(), 0, 0, 0, -1),           # weight length
        (w, 0, d.vocab, 0, -2),                 # token out of range
        (w, 0, 2 ** 32 - 1, 0, -2),             # token = -1 as u32
        (w, 0, 0, -1, -3),                      # negative position
        (w, d.max_pos * per, 0, d.max_pos, -3),  # position 128 (max_pos)
        (w, per, 0, 0, -4),                     # cache length != pos * per
        (w, 0, 0, 1, -4),
    ]
    for wt, cw, tok, pos, want in cases:
        rc, lg, c = step(wt, cw, tok, pos)
        assert rc == want, (cw, tok, pos, rc)
        assert np.all(lg == 7.0) and np.array_equal(c, cache)
    for toks, want in ((np.zeros(0, np.uint32), -2), (np.zeros(d.max_pos + 1, np.uint32), -2),
                       (np.array([0, d.vocab], np.uint32), -2)):
        lg = np.full(d.vocab, 7.0, np.float32)
        rc = lib.oracle_infer(ctypes.byref(dd), w, w.size, toks, toks.size, lg)
        assert rc == want and np.all(lg == 7.0)


@pytest.mark.parametrize("pos", [0, 5])
def test_position_zero_and_later_use_own_rows(ckpt_tiny_robust, pos):
    """cachedStep uses the supplied cache contents: changing a prior row changes the result
    (pos > 0), while a cache with the right contents reproduces the session."""
    d = synth.TINY
    toks = synth.make_tokens(9, pos + 1, d)
    lg, cache = oracle.session(d, ckpt_tiny_robust, toks)
    per = oracle.cache_words_per_pos(d)
    c = cache.copy()
    rc, again = oracle.cached_step(d, ckpt_tiny_robust, c, pos * per, int(toks[pos]), pos)
    assert rc == 0 and np.array_equal(again, lg[pos])
    if pos > 0:
        c = cache.copy()
        c[:per] += 0.5
        rc, moved = oracle.cached_step(d, ckpt_tiny_robust, c, pos * per, int(toks[pos]), pos)
        assert rc == 0 and not np.array_equal(moved, lg[pos])
