"""Closed-form sizes and layout of the packed checkpoint and the cache.

Pins: LeanExe GPT-2 README, checkpoint paragraph (124,439,808 words,
497,759,232 bytes, 1,024 position rows) and cachedStep paragraph (position x 12 x
1536 x 4 bytes; index (source*12 + layer)*1536 + offset); marXiv 2609.00018
abstract (6,432,896 logits = 128 positions x 50,257).
"""
import numpy as np

import oracle
import synth


def test_checkpoint_word_count_matches_page():
    assert oracle.ckpt_words(synth.GPT2) == 124_439_808
    assert synth.ckpt_words(synth.GPT2) == 124_439_808
    assert oracle.ckpt_words(synth.GPT2) * 4 == 497_759_232


def test_cache_row_and_session_sizes():
    per = oracle.cache_words_per_pos(synth.GPT2)
    assert per == 12 * 1536
    assert per * 4 == 73_728
    assert 128 * synth.GPT2.vocab == 6_432_896


def test_offsets_agree_between_generator_and_oracle():
    for d in (synth.GPT2, synth.TINY):
        off = synth.offsets(d)
        assert oracle.tensor_offset(d, "wte") == off["wte"][0] == 0
        assert oracle.tensor_offset(d, "wpe") == off["wpe"][0] == d.vocab * d.d_model
        assert oracle.tensor_offset(d, "lnf_g") == off["lnf_g"][0]
        assert oracle.tensor_offset(d, "lnf_b") == off["lnf_b"][0]
        for l in range(d.n_layer):
            for name in oracle.BLOCK_TENSORS:
                assert oracle.tensor_offset(d, name, l) == off[f"h{l}.{name}"][0], (l, name)


def test_block_stride_gpt2():
    d = synth.GPT2
    assert oracle.tensor_offset(d, "ln1_g", 0) == 38_597_376 + 786_432
    assert oracle.tensor_offset(d, "ln1_g", 1) - oracle.tensor_offset(d, "ln1_g", 0) == 7_087_872
    assert oracle.tensor_offset(d, "lnf_g") == 124_438_272


def test_generator_recipe():
    d = synth.TINY
    w = synth.make_checkpoint(0, d)
    off = synth.offsets(d)
    for name, (o, n) in off.items():
        t = w[o:o + n]
        if name.endswith("_g"):
            assert np.all(t == 1.0), name
        elif name.endswith("_b"):
            assert np.all(t == 0.0), name
        else:
            assert abs(float(t.std()) - 0.02) < 0.004, name
    toks = synth.make_tokens(100, 1000, d)
    assert toks.dtype == np.uint32 and toks.min() >= 0 and toks.max() < d.vocab
    assert np.array_equal(toks, synth.make_tokens(100, 1000, d))


def test_peaked_recipe():
    """The peaked variant is the plain draw with query/key columns times 10 and
    position rows 5 = 9 = 17; the tied token stream repeats a token there."""
    d = synth.TINY
    base = synth.make_checkpoint(0, d)
    pk = synth.make_checkpoint(0, d, peaked=True)
    off = synth.offsets(d)
    D = d.d_model
    for name, (o, n) in off.items():
        if name.endswith(".attn_w"):
            m0, m1 = base[o:o + n].reshape(D, 3 * D), pk[o:o + n].reshape(D, 3 * D)
            assert np.array_equal(m1[:, :2 * D], m0[:, :2 * D] * np.float32(synth.PEAK_QK_SCALE)), name
            assert np.array_equal(m1[:, 2 * D:], m0[:, 2 * D:]), name
        elif name == "wpe":
            r0, r1 = base[o:o + n].reshape(-1, D), pk[o:o + n].reshape(-1, D)
            p0 = synth.PEAK_TIED_POSITIONS[0]
            for p in range(r0.shape[0]):
                want = r0[p0] if p in synth.PEAK_TIED_POSITIONS else r0[p]
                assert np.array_equal(r1[p], want), p
        else:
            assert np.array_equal(pk[o:o + n], base[o:o + n]), name
    t = synth.make_tied_tokens(5, 20, d)
    assert t[5] == t[9] == t[17]
