"""Pins of the oracle's binary16 weight storage (gpt2.s page, options, -h).

- The rounding against numpy's float32 -> float16 conversion (an independent IEEE
  implementation) on random bit patterns and hand-worked edge cases.
- The rounded copy: exactly the 48 block matrices and the token table change.
- The whole step against transformers' GPT-2 in float64 whose block matrices and
  untied output head hold numpy-rounded values while the embedding table keeps the
  binary32 values: a matrix left unrounded, a rounded embedding or a head read from
  the wrong table moves the logits far beyond float32 rounding (the test checks
  that the rounding itself is visible at that tolerance).
"""
import numpy as np
import pytest

import hf_ref
import oracle
import synth


def test_round_binary16_matches_numpy_conversion():
    rng = np.random.default_rng(7)
    x = rng.integers(0, 2 ** 32, 400_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([x[np.isfinite(x)], rng.normal(0, 0.02, 200_000).astype(np.float32)])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float32)
    got = oracle.round_binary16(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("x,want", [
    (65504.0, 65504.0),                     # largest binary16
    (65519.99, 65504.0),                    # below the midpoint to 2^16
    (65520.0, np.inf),                      # the midpoint rounds to even = 2^16: overflow
    (1.0 + 2.0 ** -11, 1.0),                # tie between 1 and 1 + 2^-10: even is 1
    (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),  # tie between 1+2^-10 and 1+2^-9: even is 1+2^-9
    (2.0 ** -24, 2.0 ** -24),               # smallest subnormal
    (2.0 ** -25, 0.0),                      # tie between 0 and 2^-24: even is 0
    (3 * 2.0 ** -26, 2.0 ** -24),           # above that tie
    (2.0 ** -14 - 2.0 ** -25, 2.0 ** -14),  # tie at the subnormal/normal boundary: even is 2^-14
    (-0.0, -0.0),
    (-65520.0, -np.inf),
])
def test_round_binary16_hand_cases(x, want):
    got = oracle.round_binary16(np.array([x], np.float32))[0]
    assert np.float32(want).view(np.uint32) == got.view(np.uint32)


def test_f16_weights_round_exactly_the_matrices(ckpt_tiny_robust):
    d = synth.TINY
    w = ckpt_tiny_robust
    w16 = oracle.f16_weights(d, w)
    changed = np.zeros(w.size, bool)
    for name, (o, n) in synth.offsets(d).items():
        if name == "wte" or name.endswith("_w"):
            assert np.array_equal(w16[o:o + n], w[o:o + n].astype(np.float16).astype(np.float32)), name
            changed[o:o + n] = True
    assert np.array_equal(w16[~changed], w[~changed])
    assert not np.array_equal(w16[changed], w[changed])


def test_tiny_f16_session_matches_transformers(ckpt_tiny_robust):
    d = synth.TINY
    w = ckpt_tiny_robust
    toks = synth.make_tokens(5, d.max_pos, d)
    lg, _ = oracle.session(d, w, toks, f16=oracle.f16_weights(d, w))
    ref = hf_ref.logits_all_positions(hf_ref.build(w, d, f16=True), toks)
    tol = 2e-6 * max(1.0, np.abs(ref).max())
    assert np.abs(ref - lg).max() <= tol
    # the rounding is visible at this tolerance: the fp32 step is far from it
    lg32, _ = oracle.session(d, w, toks)
    assert np.abs(lg32 - ref).max() > 20 * tol


@pytest.mark.slow
def test_gpt2_seed0_f16_eight_steps_match_transformers(ckpt_gpt2):
    d = synth.GPT2
    toks = synth.make_tokens(synth.SEED_SHORT, 8, d)
    lg, _ = oracle.session(d, ckpt_gpt2, toks, f16=oracle.f16_weights(d, ckpt_gpt2))
    ref = hf_ref.logits_all_positions(hf_ref.build(ckpt_gpt2, d, f16=True), toks)
    assert np.abs(ref - lg).max() <= 5e-5
    lg32, _ = oracle.session(d, ckpt_gpt2, toks)
    assert np.abs(lg32 - ref).max() > 4 * 5e-5
