"""The C-ABI library loads without a GPU, exports every symbol include/gpt2.h
declares, and rejects invalid scalar arguments on the host (LeanExe GPT-2 README:
invalid weight length, token, position or cache length give empty results;
marXiv 2609.00018 abstract: sessions of at most 128 tokens).  No call here reaches
a kernel: every argument set is one the host validation refuses."""
import ctypes
import os
import re

import pytest

import stream_gpt_transformer_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gpt2.h")

if not os.path.exists(g.LIB_PATH):
    pytest.skip("libgpt2mi.so not built (run __graft_entry__.build())", allow_module_level=True)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gpt2_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) >= 14
    L = ctypes.CDLL(g.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
        assert n in g.SIGNATURES, n
    assert set(g.SIGNATURES) == set(names)


def test_sizes():
    assert g.gpt2_packed_nbytes(0) == 0 and g.gpt2_packed_nbytes(8) == 0
    f32 = g.gpt2_packed_nbytes(g.GPT2_PACK_F32)
    f16 = g.gpt2_packed_nbytes(g.GPT2_PACK_F16)
    # binary16: the block matrices and the token table at two bytes each (besides the
    # fp32 token table and position rows every form keeps)
    assert 0 <= f16 - (f32 - 12 * 7_077_888 * 4) - (12 * 7_077_888 + 50257 * 768) * 2 < 4096
    assert g.gpt2_packed_nbytes(7) > g.gpt2_packed_nbytes(3)
    q8 = g.gpt2_packed_nbytes(g.GPT2_PACK_Q8)
    both = g.gpt2_packed_nbytes(3)
    # fp32 [out][in] block matrices: 12 x 7,077,888 words; int8: the same count of bytes
    # plus the 50,257 x 768 head and one fp32 scale per 64 codes.
    assert f32 - q8 > 12 * 7_077_888 * 4 - (12 * 7_077_888 + 50257 * 768) * (1 + 4 / 64) - 4096
    assert both > f32 and both > q8
    assert g.gpt2_workspace_nbytes() > 64 * (768 * 3 + 2304 + 3072) * 4
    assert g.gpt2_q8_capture_nbytes() > 50257 * 12 * 4


def test_capture_offsets_are_ordered_and_disjoint():
    prev_end = 0
    for layer in range(12):
        for m in range(4):
            o = g.gpt2_q8_capture_offsets(layer, m)
            assert o["base"] >= prev_end
            assert o["base"] <= o["in"] < o["codes"] < o["scales"] < o["acc"] < o["out"]
            prev_end = o["out"]
    h = g.gpt2_q8_capture_offsets(0, 4)
    assert h["base"] >= prev_end
    assert h["out"] + 50257 * 4 <= g.gpt2_q8_capture_nbytes()
    with pytest.raises(g.Gpt2Error):
        g.gpt2_q8_capture_offsets(12, 0)


FAKE = 0x10000  # a 16-byte-aligned address that validation never dereferences


def test_pack_validation():
    n = g.gpt2_packed_nbytes(3)
    assert g.gpt2_pack_weights(FAKE, g.GPT2_CKPT_BYTES - 4, FAKE, n, 3)[0] == g.GPT2_EWEIGHTS
    assert g.gpt2_pack_weights(0, g.GPT2_CKPT_BYTES, FAKE, n, 3)[0] == g.GPT2_EWEIGHTS
    assert g.gpt2_pack_weights(FAKE, g.GPT2_CKPT_BYTES, FAKE, n - 1, 3)[0] == g.GPT2_EARG
    assert g.gpt2_pack_weights(FAKE, g.GPT2_CKPT_BYTES, FAKE, n, 0)[0] == g.GPT2_EARG
    assert g.gpt2_pack_weights(FAKE + 4, g.GPT2_CKPT_BYTES, FAKE, n, 3)[0] == g.GPT2_EARG


def test_step_validation_without_model():
    for fn in (g.gpt2_cached_step, g.gpt2_q8_cached_step, g.gpt2_f16_cached_step):
        assert fn(None, FAKE, 0, 0, 0, FAKE, FAKE) == g.GPT2_EARG
    for grp in (64, 0, 384):
        assert g.gpt2_q8_cached_step_grouped(None, grp, FAKE, 0, 0, 0, FAKE, FAKE) == g.GPT2_EARG
    assert g.gpt2_q8_cached_step_grouped(None, 96, FAKE, 0, 0, 0, FAKE, FAKE) == g.GPT2_EARG
    assert g.gpt2_q8_weight_group(None) == -1
    # an invalid weight group is rejected before any device work
    for grp in (32, 96, 1536, 3072, -64):
        rc, h = g.gpt2_pack_weights_grouped(FAKE, g.GPT2_CKPT_BYTES, FAKE, 1 << 40, g.GPT2_PACK_Q8, grp)
        assert rc == g.GPT2_EARG and h is None
    assert g.gpt2_cached_step_noalloc(None, FAKE, 0, 0, 0, FAKE) == g.GPT2_EARG
    assert g.gpt2_infer(None, [1, 2], FAKE, FAKE) == g.GPT2_EARG
    assert g.gpt2_batched_cached_step(None, FAKE, 18432, [0], [0], [0], FAKE, FAKE) == g.GPT2_EARG


def test_test_hook_validation():
    assert g.gpt2_test_quantize(FAKE, 65, FAKE, FAKE) == g.GPT2_EARG
    assert g.gpt2_test_quantize(FAKE, -64, FAKE, FAKE) == g.GPT2_EARG
    assert g.gpt2_test_gemm(FAKE, FAKE, FAKE, 0, 64, 32) == g.GPT2_EARG
    assert g.gpt2_test_gemm(FAKE, FAKE, FAKE, 129, 64, 32) == g.GPT2_EARG
    assert g.gpt2_test_gemm(FAKE, FAKE, FAKE, 8, 65, 32) == g.GPT2_EARG
    assert g.gpt2_test_gemm(FAKE, FAKE, FAKE, 8, 64, 33) == g.GPT2_EARG
    assert g.gpt2_test_gemm_bias(FAKE, FAKE, FAKE, FAKE, 8, 24, 32, 0) == g.GPT2_EARG
    assert g.gpt2_test_gemm_bias(FAKE, FAKE, FAKE, FAKE, 8, 32, 48, 0) == g.GPT2_EARG
    assert g.gpt2_test_gemm_bias(FAKE, FAKE, FAKE, FAKE, 8, 32, 64, 2) == g.GPT2_EARG
    assert g.gpt2_test_layernorm_seq(FAKE, -1, FAKE, FAKE, FAKE) == g.GPT2_EARG
    assert g.gpt2_test_layernorm_seq(0, 2, FAKE, FAKE, FAKE) == g.GPT2_EARG


def test_prefill_validation_without_model():
    assert g.gpt2_prefill(None, [1, 2], FAKE, 2 * g.GPT2_CACHE_WORDS_PER_POS, FAKE, FAKE) == g.GPT2_EARG


def test_generate_validation_without_model():
    assert g.gpt2_generate(None, FAKE, 20 * g.GPT2_CACHE_WORDS_PER_POS, [1, 2], 4, 0, FAKE, FAKE, FAKE, FAKE) == g.GPT2_EARG
