"""Pins of the oracle's int8 granularity variants (marXiv 2609.00018 abstract).

Weight scales per group of gw inputs of an output row, input scales per group of gx
coordinates (0 = the whole row); integer sums over the gcd(gx, gw) groups on which
both scales are constant.

- gw = gx = 64 is the group-64 path, bit for bit (weights and whole sessions).
- The storage the abstract prints (74.3 % smaller) follows from one weight scale
  per output row, and not from one per 64 inputs.
- On the code grid (values k * 2^e with a +-127 anchor in each group) every step of
  a variant projection is exact, so it equals the float64 product: a wrong group
  index, a wrong gcd or a scale taken from the wrong group breaks equality.
- Whole sessions against a float64 forward with the oracle's dequantized weights and
  fake-quantized inputs, for each variant, on a model wide enough (768 / 3,072-wide
  is not needed: d_model 256, d_ff 1024) that row and group scales differ.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

MID = synth.Dims(n_layer=2, d_model=256, n_head=4, d_ff=1024, vocab=97, n_pos_rows=40, max_pos=32)


def test_group64_variant_is_the_group64_path(ckpt_tiny_robust):
    d = synth.TINY
    w = ckpt_tiny_robust
    c64, s64 = oracle.q8_quantize_weights(d, w)
    c, s = oracle.qv_quantize_weights(d, w, 64)
    assert np.array_equal(c, c64) and np.array_equal(s, s64)
    toks = synth.make_tokens(6, 12, d)
    a, ca = oracle.session(d, w, toks, q8=(c64, s64))
    b, cb = oracle.qv_session(d, w, toks, 64, 64, (c, s))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(ca.view(np.uint32), cb.view(np.uint32))


def test_row_weight_scales_give_the_published_storage_reduction():
    """int8 codes of the 48 matrices and the token table, binary32 scales, and the
    binary32 position table (all 1,024 rows), LayerNorm parameters and biases: one
    scale per output row gives 74.3 % less than the 497,759,232-byte checkpoint (the
    abstract's figure); one per 64 inputs gives 72.9 %."""
    d = synth.GPT2
    off = synth.offsets(d)
    rest = sum(n for name, (o, n) in off.items() if name != "wte" and not name.endswith("_w"))
    total = synth.ckpt_words(d) * 4
    red = {}
    for gw in (0, 64):
        nc, ns = oracle.qv_sizes(d, gw)
        red[gw] = 1 - (nc + 4 * ns + 4 * rest) / total
    assert round(red[0] * 100, 1) == 74.3
    assert round(red[64] * 100, 1) == 72.9


def _grid(rng, K, G, small=4):
    """K values k * 2^e, |k| <= small, with one +-127 anchor per group of G (so the
    group's scale is exactly 2^e) and e in -3..0 per group."""
    v = rng.integers(-small, small + 1, K).astype(np.float64)
    ng = K // G
    e = rng.integers(-3, 1, ng).astype(np.float64)
    for g in range(ng):
        v[g * G + rng.integers(0, G)] = 127 * rng.choice([-1, 1])
    return v * np.repeat(2.0 ** e, G)


@pytest.mark.parametrize("K,gx,gw", [(768, 0, 0), (768, 64, 0), (768, 0, 64), (768, 128, 192),
                                     (768, 256, 384), (3072, 0, 0), (3072, 768, 64), (3072, 192, 0),
                                     (3072, 384, 256)])
def test_lossless_grid_variant_projection_is_exact(K, gx, gw):
    rng = np.random.default_rng(K + 7 * gx + 13 * gw)
    N = 24
    GX, GW = gx or K, gw or K
    x = _grid(rng, K, GX).astype(np.float32)
    W = np.stack([_grid(rng, K, GW) for _ in range(N)])
    b = (rng.integers(-8, 9, N) * 0.25).astype(np.float32)
    # the weights through the oracle's variant quantizer: place W^T as the MLP
    # projection ([in][out], K = d_ff inputs) or the token table (K = d_model)
    if K == 3072:
        d = synth.Dims(n_layer=1, d_model=768, n_head=12, d_ff=3072, vocab=64, n_pos_rows=2, max_pos=2)
        w = np.zeros(synth.ckpt_words(d), np.float32)
        o, n = synth.offsets(d)["h0.mlpproj_w"]
        Wfull = np.zeros((3072, 768))
        Wfull[:, :N] = W.T
        w[o:o + n] = Wfull.astype(np.float32).reshape(-1)
        codes, scales = oracle.qv_quantize_weights(d, w, gw)
        # layer 0 matrices in order: attn [2304][768], attnproj [768][768], fc [3072][768], mlpproj [768][3072]
        co = 2304 * 768 + 768 * 768 + 3072 * 768
        so = sum(r * (k // (gw or k)) for r, k in ((2304, 768), (768, 768), (3072, 768)))
        nsr = K // GW
        wc = codes[co:co + 768 * K].reshape(768, K)[:N]
        ws = scales[so:so + 768 * nsr].reshape(768, nsr)[:N]
    else:
        d = synth.Dims(n_layer=1, d_model=768, n_head=12, d_ff=3072, vocab=N, n_pos_rows=2, max_pos=2)
        w = np.zeros(synth.ckpt_words(d), np.float32)
        o, n = synth.offsets(d)["wte"]
        w[o:o + n] = W.astype(np.float32).reshape(-1)
        codes, scales = oracle.qv_quantize_weights(d, w, gw)
        nc, ns = oracle.qv_sizes(d, gw)
        wc = codes[nc - N * K:].reshape(N, K)
        ws = scales[ns - N * (K // GW):].reshape(N, K // GW)
    assert np.array_equal(wc.astype(np.float64) * np.repeat(ws, GW, 1), W)
    xc, xs, acc, y = oracle.qv_linear(x, gx, wc, ws, gw, b)
    assert np.array_equal(xc.astype(np.float64) * np.repeat(xs, GX), x.astype(np.float64))
    GM = math.gcd(GX, GW)
    assert acc.shape == (N, K // GM)
    assert np.array_equal(acc, (wc.astype(np.int64) * xc.astype(np.int64)).reshape(N, K // GM, GM).sum(2))
    assert np.array_equal(y.astype(np.float64), W @ x.astype(np.float64) + b)


def test_zero_and_tiny_groups():
    """An all-zero input group has scale 0 and codes 0 and adds nothing; a group whose
    largest magnitude is subnormal still gets a scale from max/127."""
    K = 768
    rng = np.random.default_rng(3)
    x = rng.standard_normal(K).astype(np.float32)
    x[128:256] = 0.0
    wc = rng.integers(-127, 128, (3, K)).astype(np.int8)
    ws = np.full((3, K // 128), 0.01, np.float32)
    xc, xs, acc, y = oracle.qv_linear(x, 128, wc, ws, 128)
    assert xs[1] == 0 and not xc[128:256].any() and not acc[:, 1].any()
    x2 = np.zeros(K, np.float32)
    x2[5] = np.float32(1e-40)
    xc2, xs2, _, _ = oracle.qv_linear(x2, 0, wc, np.full((3, 1), 0.01, np.float32), 0)
    assert xs2[0] == np.float32(np.float32(1e-40) / np.float32(127)) and xc2[5] == 127


def _fake_quant(x: torch.Tensor, G: int) -> torch.Tensor:
    g = x.reshape(-1, G)
    s = g.abs().amax(1, keepdim=True) / 127
    c = torch.where(s > 0, torch.round(g / torch.where(s > 0, s, torch.ones_like(s))), torch.zeros_like(g))
    return (c.clamp(-127, 127) * s).reshape(x.shape)


def _reference_session(d, w, codes, scales, gw, gx, toks):
    """float64 forward with the oracle's variant weight codes dequantized and inputs
    fake-quantized in groups of gx (torch.round is half-to-even)."""
    D, F, H = d.d_model, d.d_ff, d.n_head
    dh = D // H
    off = synth.offsets(d)
    # the variant store: per layer attn [3D][D], attnproj [D][D], fc [F][D], mlpproj [D][F], then the head
    shapes = [(3 * D, D), (D, D), (F, D), (D, F)]
    co, so, offs = 0, 0, {}
    for l in range(d.n_layer):
        for name, (N, K) in zip(("attn_w", "attnproj_w", "fc_w", "mlpproj_w"), shapes):
            offs[(l, name)] = (co, so, N, K)
            co += N * K
            so += N * (K // (gw or K))
    offs[(0, "head")] = (co, so, d.vocab, D)

    def t(name, shape):
        o, n = off[name]
        return torch.from_numpy(w[o:o + n].astype(np.float64).reshape(shape))

    def deq(l, m):
        c0, s0, N, K = offs[(l, m)]
        G = gw or K
        c = torch.from_numpy(codes[c0:c0 + N * K].astype(np.float64).reshape(N, K))
        s = torch.from_numpy(scales[s0:s0 + N * (K // G)].astype(np.float64).reshape(N, K // G))
        return c * s.repeat_interleave(G, 1)

    def fq(rows):
        return torch.stack([_fake_quant(r, gx or r.numel()) for r in rows])

    def ln(x, g, b):
        return torch.nn.functional.layer_norm(x, (D,), g, b, eps=1e-5)

    T = len(toks)
    X = t("wte", (d.vocab, D))[torch.from_numpy(toks.astype(np.int64))] + t("wpe", (d.n_pos_rows, D))[:T]
    for l in range(d.n_layer):
        h = ln(X, t(f"h{l}.ln1_g", (D,)), t(f"h{l}.ln1_b", (D,)))
        qkv = fq(h) @ deq(l, "attn_w").T + t(f"h{l}.attn_b", (3 * D,))
        q, k, v = (z.reshape(T, H, dh).transpose(0, 1) for z in qkv.split(D, 1))
        a = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(0, 1).reshape(T, D)
        X = X + fq(a) @ deq(l, "attnproj_w").T + t(f"h{l}.attnproj_b", (D,))
        h = ln(X, t(f"h{l}.ln2_g", (D,)), t(f"h{l}.ln2_b", (D,)))
        u = fq(h) @ deq(l, "fc_w").T + t(f"h{l}.fc_b", (F,))
        g = torch.nn.functional.gelu(u, approximate="tanh")
        X = X + fq(g) @ deq(l, "mlpproj_w").T + t(f"h{l}.mlpproj_b", (D,))
    h = ln(X, t("lnf_g", (D,)), t("lnf_b", (D,)))
    return (fq(h) @ deq(0, "head").T).numpy()


@pytest.mark.parametrize("gw,gx", [(0, 0), (0, 64), (64, 0), (128, 256), (256, 128)])
def test_variant_session_matches_float64_fake_quant(gw, gx):
    d = MID
    w = synth.make_checkpoint(9, d, robust=True)
    codes, scales = oracle.qv_quantize_weights(d, w, gw)
    toks = synth.make_tokens(8, 12, d)
    lg, _ = oracle.qv_session(d, w, toks, gw, gx, (codes, scales))
    ref = _reference_session(d, w, codes, scales, gw, gx, toks)
    diff = np.abs(lg - ref)
    # float32 against float64; a rare input code may round the other way
    assert np.median(diff) <= 1e-6
    assert diff.max() <= 2e-3
    # the variants are distinct computations
    if (gw, gx) != (64, 64):
        c64, s64 = oracle.q8_quantize_weights(d, w)
        l64, _ = oracle.session(d, w, toks, q8=(c64, s64))
        assert np.abs(l64 - lg).max() > 1e-4


def test_variant_rejects_bad_groups():
    d = synth.GPT2
    for g in (32, 100, 320, 1536, -64):
        c, s = oracle._sz(), oracle._sz()
        import ctypes
        assert oracle.lib().oracle_qv_sizes(ctypes.byref(oracle.dims(d)), g, ctypes.byref(c), ctypes.byref(s)) != 0
