"""Pins of the int8 group-64 path of the oracle (marXiv 2609.00018 abstract:
signed eight-bit weights and projection inputs, 32-bit integer accumulation,
binary32 elsewhere; scales per consecutive group of 64 coordinates; nearest-even
rounding; saturation; a fixed rescale order).

- Hand-worked code cases with power-of-two scales (tests/golden/quantizer_cases.txt).
- Properties of the rule on random groups: the extreme value codes to +-127,
  every code is within half a step of x/s, codes stay in [-127, 127].
- Group accumulators against exact integer arithmetic.
- A lossless case (values on the code grid, power-of-two scales, small sums): the
  quantized projection must equal the exact float64 product bit for bit.
- The whole quantized step against a float64 fake-quant forward of the tiny model.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import golden_path


def _golden():
    groups, scaled = [], []
    with open(golden_path("quantizer_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = [p.strip() for p in line.split("|")]
            if parts[0] == "group":
                _, name, anchor, vals, codes, scale = parts
                groups.append((name, float(anchor), [float(v) for v in vals.split()],
                               [int(c) for c in codes.split()], float(scale)))
            elif parts[0] == "scaled":
                _, name, s, vals, codes = parts
                scaled.append((name, float(s), [float(v) for v in vals.split()],
                               [int(c) for c in codes.split()]))
    return groups, scaled


GROUPS, SCALED = _golden()


@pytest.mark.parametrize("case", GROUPS, ids=[c[0] for c in GROUPS])
def test_golden_group_cases(case):
    name, anchor, vals, want, want_s = case
    x = np.zeros(64, np.float32)
    x[:len(vals)] = vals
    x[63] = anchor
    codes, scales = oracle.quantize(x)
    assert scales[0] == np.float32(want_s)
    assert list(codes[:len(vals)]) == want
    assert np.all(codes[len(vals):63] == 0)


@pytest.mark.parametrize("case", SCALED, ids=[c[0] for c in SCALED])
def test_golden_scaled_cases(case):
    name, s, vals, want = case
    codes = oracle.quantize_with_scale(np.array(vals, np.float32), s)
    assert list(codes) == want


def test_random_group_properties():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(64 * 400) * np.repeat(10.0 ** rng.uniform(-3, 3, 400), 64)).astype(np.float32)
    codes, scales = oracle.quantize(x)
    xg = x.reshape(400, 64).astype(np.float64)
    cg = codes.reshape(400, 64).astype(np.float64)
    s = scales.astype(np.float64)
    m = np.abs(xg).max(1)
    assert np.all(np.abs(s - m / 127) <= 2 ** -24 * m / 127 * 1.0001)
    assert np.all(np.abs(cg) <= 127)
    # the largest |x| of each group codes to +-127 with its sign
    i = np.abs(xg).argmax(1)
    assert np.all(cg[np.arange(400), i] == 127 * np.sign(xg[np.arange(400), i]))
    # each code within half a step (plus the rounding of x/s) of x/s
    r = xg / s[:, None]
    assert np.all(np.abs(cg - r) <= 0.5 + 1e-4)
    # strictly closer than half a step means the nearest integer
    far = np.abs(np.abs(r - np.floor(r)) - 0.5) > 1e-3
    assert np.all(cg[far] == np.round(r[far]))


def test_accumulators_are_exact_integers():
    rng = np.random.default_rng(1)
    K, N = 768, 50
    wc = rng.integers(-127, 128, (N, K)).astype(np.int8)
    ws = rng.uniform(1e-4, 1e-2, (N, K // 64)).astype(np.float32)
    xc = rng.integers(-127, 128, K).astype(np.int8)
    xs = rng.uniform(1e-3, 1e-1, K // 64).astype(np.float32)
    acc, y = oracle.q8_linear_codes(xc, xs, wc, ws)
    ref = (wc.astype(np.int64).reshape(N, K // 64, 64) * xc.astype(np.int64).reshape(K // 64, 64)).sum(2)
    assert np.array_equal(acc.astype(np.int64), ref)
    # extreme accumulators stay exact: all codes +-127
    wc[:] = 127
    xc[:] = -127
    acc, _ = oracle.q8_linear_codes(xc, xs, wc, ws)
    assert np.all(acc == -64 * 127 * 127)

    # the rescale weights each group by its own row and input scales: within the
    # float32 error of a 12-term sum of 2-product terms of the exact float64 value
    wc = rng.integers(-127, 128, (N, K)).astype(np.int8)
    xc = rng.integers(-127, 128, K).astype(np.int8)
    acc, y = oracle.q8_linear_codes(xc, xs, wc, ws)
    terms = acc.astype(np.float64) * ws.astype(np.float64) * xs.astype(np.float64)
    bound = (K // 64 + 2) * 2.0 ** -24 * np.abs(terms).sum(1)
    assert np.all(np.abs(y - terms.sum(1)) <= bound)


def _grid_group_values(rng, n_groups, exps, small=16):
    """Values k * 2^e with |k| <= small, one +-127 anchor per group (so s = 2^e exactly)."""
    v = rng.integers(-small, small + 1, (n_groups, 64)).astype(np.float64)
    v[np.arange(n_groups), rng.integers(0, 64, n_groups)] = 127 * rng.choice([-1, 1], n_groups)
    return v * (2.0 ** exps)[:, None]


def test_lossless_grid_projection_is_exact():
    """On the code grid every step of the quantized projection is exact, so the result must
    equal the float64 product exactly; a wrong group index, a transposed operand or a missing
    scale breaks equality."""
    rng = np.random.default_rng(2)
    K, N = 768, 40
    G = K // 64
    xe = rng.integers(-3, 1, G).astype(np.float64)
    x = _grid_group_values(rng, G, xe).reshape(K).astype(np.float32)
    W = np.zeros((N, K))
    for j in range(N):
        W[j] = _grid_group_values(rng, G, rng.integers(-3, 1, G).astype(np.float64)).reshape(K)
    b = (rng.integers(-8, 9, N) * 0.25).astype(np.float32)
    # weights through the oracle's weight quantizer (checkpoint layout [in][out])
    d = synth.Dims(n_layer=1, d_model=K, n_head=12, d_ff=64 * 2, vocab=N, n_pos_rows=2, max_pos=2)
    w = np.zeros(synth.ckpt_words(d), np.float32)
    o, n = synth.offsets(d)["wte"]
    w[o:o + n] = W.astype(np.float32).reshape(-1)
    codes, scales = oracle.q8_quantize_weights(d, w)
    co, so = oracle.q8_offsets(d, 0, "head")
    wc = codes[co:co + N * K].reshape(N, K)
    ws = scales[so:so + N * G].reshape(N, G)
    assert np.array_equal(wc.astype(np.float64) * np.repeat(ws, 64, 1), W)
    xc, xs, acc, y = oracle.q8_linear(x, wc, ws, b)
    assert np.array_equal(xc.astype(np.float64) * np.repeat(xs, 64), x.astype(np.float64))
    exact = W @ x.astype(np.float64) + b
    assert np.array_equal(y.astype(np.float64), exact)


def test_weight_codes_follow_checkpoint_columns():
    """Row j, group g of a block matrix quantizes inputs 64g..64g+63 of output j, i.e. the
    checkpoint column W[64g:64g+64, j] of the [in][out] matrix."""
    d = synth.TINY
    w = synth.make_checkpoint(4, d, robust=True)
    codes, scales = oracle.q8_quantize_weights(d, w)
    off = synth.offsets(d)
    D, F = d.d_model, d.d_ff
    for l in range(d.n_layer):
        for name, (K, N) in (("attn_w", (D, 3 * D)), ("attnproj_w", (D, D)), ("fc_w", (D, F)),
                             ("mlpproj_w", (F, D))):
            o, n = off[f"h{l}.{name}"]
            W = w[o:o + n].reshape(K, N)
            co, so = oracle.q8_offsets(d, l, name)
            wc = codes[co:co + N * K].reshape(N, K)
            ws = scales[so:so + N * (K // 64)].reshape(N, K // 64)
            for j in (0, N // 3, N - 1):
                c, s = oracle.quantize(np.ascontiguousarray(W[:, j]))
                assert np.array_equal(wc[j], c) and np.array_equal(ws[j], s), (l, name, j)


def _fake_quant(x: torch.Tensor) -> torch.Tensor:
    """float64 group-64 quantize-dequantize of activations (torch.round is half-to-even)."""
    g = x.reshape(-1, 64)
    s = g.abs().amax(1, keepdim=True) / 127
    c = torch.where(s > 0, torch.round(g / torch.where(s > 0, s, torch.ones_like(s))), torch.zeros_like(g))
    return (c.clamp(-127, 127) * s).reshape(x.shape)


def _q8_reference_session(d, w, codes, scales, toks):
    """float64 forward with the oracle's weight codes dequantized and fake-quantized inputs."""
    D, F, H = d.d_model, d.d_ff, d.n_head
    dh = D // H
    off = synth.offsets(d)

    def t(name, shape):
        o, n = off[name]
        return torch.from_numpy(w[o:o + n].astype(np.float64).reshape(shape))

    def deq(l, m, N, K):
        co, so = oracle.q8_offsets(d, l, m)
        c = torch.from_numpy(codes[co:co + N * K].astype(np.float64).reshape(N, K))
        s = torch.from_numpy(scales[so:so + N * (K // 64)].astype(np.float64).reshape(N, K // 64))
        return c * s.repeat_interleave(64, 1)

    def ln(x, g, b):
        return torch.nn.functional.layer_norm(x, (D,), g, b, eps=1e-5)

    T = len(toks)
    X = t("wte", (d.vocab, D))[torch.from_numpy(toks.astype(np.int64))] + t("wpe", (d.n_pos_rows, D))[:T]
    for l in range(d.n_layer):
        Wq = deq(l, "attn_w", 3 * D, D)
        h = ln(X, t(f"h{l}.ln1_g", (D,)), t(f"h{l}.ln1_b", (D,)))
        qkv = torch.stack([_fake_quant(r) for r in h]) @ Wq.T + t(f"h{l}.attn_b", (3 * D,))
        q, k, v = qkv.split(D, 1)
        q = q.reshape(T, H, dh).transpose(0, 1)
        k = k.reshape(T, H, dh).transpose(0, 1)
        v = v.reshape(T, H, dh).transpose(0, 1)
        a = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
        a = a.transpose(0, 1).reshape(T, D)
        X = X + torch.stack([_fake_quant(r) for r in a]) @ deq(l, "attnproj_w", D, D).T + t(f"h{l}.attnproj_b", (D,))
        h = ln(X, t(f"h{l}.ln2_g", (D,)), t(f"h{l}.ln2_b", (D,)))
        u = torch.stack([_fake_quant(r) for r in h]) @ deq(l, "fc_w", F, D).T + t(f"h{l}.fc_b", (F,))
        g = torch.nn.functional.gelu(u, approximate="tanh")
        X = X + torch.stack([_fake_quant(r) for r in g]) @ deq(l, "mlpproj_w", D, F).T + t(f"h{l}.mlpproj_b", (D,))
    h = ln(X, t("lnf_g", (D,)), t("lnf_b", (D,)))
    return (torch.stack([_fake_quant(r) for r in h]) @ deq(0, "head", d.vocab, D).T).numpy()


def test_q8_session_matches_float64_fake_quant(ckpt_tiny_robust):
    d = synth.TINY
    w = ckpt_tiny_robust
    codes, scales = oracle.q8_quantize_weights(d, w)
    toks = synth.make_tokens(6, 16, d)
    lg, _ = oracle.session(d, w, toks, q8=(codes, scales))
    ref = _q8_reference_session(d, w, codes, scales, toks)
    diff = np.abs(lg - ref)
    # float32 vs float64 arithmetic; a rare activation code may round the other way,
    # which moves a logit by about one code step times a weight scale.
    assert np.median(diff) <= 1e-6
    assert diff.max() <= 2e-3
    # and the quantized path stays close to binary32 (diagnostic sanity)
    lf, _ = oracle.session(d, w, toks)
    assert np.abs(lf - lg).max() < 0.05


def test_q8_rejects_like_fp32(ckpt_tiny_robust):
    d = synth.TINY
    codes, scales = oracle.q8_quantize_weights(d, ckpt_tiny_robust)
    per = oracle.cache_words_per_pos(d)
    cache = np.zeros(2 * per, np.float32)
    rc, _ = oracle.q8_cached_step(d, ckpt_tiny_robust, codes, scales, cache, per, d.vocab, 1)
    assert rc == -2
    rc, _ = oracle.q8_cached_step(d, ckpt_tiny_robust, codes, scales, cache, 0, 0, 1)
    assert rc == -4
