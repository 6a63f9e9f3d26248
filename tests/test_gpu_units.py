"""GPU unit parity: packed weights, int8 weight codes, the group-64 quantizer and the
prefill matrix-core GEMM, each against the oracle or exact arithmetic."""
import numpy as np
import pytest
import torch

import oracle
import stream_gpt_transformer_amd as g
import synth
from conftest import golden_path
from gpu_common import D, checkpoint, model, need_gpu, oracle_q8

pytestmark = pytest.mark.gpu


def _dev_slice(m: g.Model, ptr: int, nbytes: int) -> torch.Tensor:
    off = ptr - m.packed.data_ptr()
    assert 0 <= off and off + nbytes <= m.packed.numel()
    return m.packed[off:off + nbytes]


def test_fp32_pack_is_transpose_of_checkpoint():
    need_gpu()
    m = model()
    w = checkpoint()
    off = synth.offsets(D)
    names = ["attn_w", "attnproj_w", "fc_w", "mlpproj_w"]
    for layer in (0, 5, 11):
        for mi, name in enumerate(names):
            v = g.gpt2_weight_view(m.handle, layer, mi)
            rows, cols = v["rows"], v["cols"]
            got = _dev_slice(m, v["f32"], rows * cols * 4).view(torch.float32).cpu().numpy().reshape(rows, cols)
            o, n = off[f"h{layer}.{name}"]
            ref = w[o:o + n].reshape(cols, rows).T
            assert np.array_equal(got, ref), (layer, name)
    v = g.gpt2_weight_view(m.handle, 0, 4)
    got = _dev_slice(m, v["f32"], v["rows"] * v["cols"] * 4).view(torch.float32).cpu().numpy()
    o, n = off["wte"]
    assert np.array_equal(got, w[o:o + n])


def test_q8_weight_codes_and_scales_bit_exact():
    """Every int8 code and group scale of the 48 block matrices and the head equals the
    oracle's quantization of the same fp32 weights."""
    need_gpu()
    m = model()
    codes, scales = oracle_q8()
    for layer in range(12):
        for mi, name in enumerate(oracle.MATRICES):
            if mi == 4 and layer > 0:
                continue
            v = g.gpt2_weight_view(m.handle, layer, mi)
            rows, cols = v["rows"], v["cols"]
            G = cols // 64
            gc = _dev_slice(m, v["codes"], rows * cols).view(torch.int8).cpu().numpy()
            gs = _dev_slice(m, v["scales"], rows * G * 4).view(torch.float32).cpu().numpy()
            co, so = oracle.q8_offsets(D, layer, name)
            assert np.array_equal(gc, codes[co:co + rows * cols]), (layer, name)
            assert np.array_equal(gs.view(np.uint32), scales[so:so + rows * G].view(np.uint32)), (layer, name)


def _gpu_quantize(x: np.ndarray):
    xd = torch.from_numpy(x).cuda()
    c = torch.empty(x.size, dtype=torch.int8, device="cuda")
    s = torch.empty(x.size // 64, dtype=torch.float32, device="cuda")
    assert g.gpt2_test_quantize(xd.data_ptr(), x.size, c.data_ptr(), s.data_ptr(), 0) == 0
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def test_quantizer_golden_cases_on_gpu():
    need_gpu()
    rows = []
    with open(golden_path("quantizer_cases.txt")) as f:
        for line in f:
            p = [t.strip() for t in line.split("|")]
            if p[0] == "group":
                rows.append((float(p[2]), [float(v) for v in p[3].split()], [int(c) for c in p[4].split()],
                             float(p[5])))
    x = np.zeros(64 * len(rows), np.float32)
    for i, (anchor, vals, _, _) in enumerate(rows):
        x[64 * i:64 * i + len(vals)] = vals
        x[64 * i + 63] = anchor
    c, s = _gpu_quantize(x)
    for i, (_, vals, want, want_s) in enumerate(rows):
        assert list(c[64 * i:64 * i + len(vals)]) == want
        assert s[i] == np.float32(want_s)


def test_quantizer_matches_oracle_bit_exact():
    need_gpu()
    rng = np.random.default_rng(11)
    G = 4096
    scale = np.repeat(10.0 ** rng.uniform(-4, 3, G), 64)
    x = (rng.standard_normal(64 * G) * scale).astype(np.float32)
    # groups with values on exact half-steps (ties) and zero groups
    k = rng.integers(-254, 255, (512, 64))
    k[:, 0] = 254
    x[:512 * 64] = (k.reshape(-1) * 0.5 * 2.0 ** rng.integers(-8, 8, 512).repeat(64)).astype(np.float32)
    x[-64 * 8:] = 0
    c, s = _gpu_quantize(x)
    oc, os_ = oracle.quantize(x)
    assert np.array_equal(c, oc)
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32))
    assert g.gpt2_test_quantize(0, 0, 0, 0, 0) == 0  # empty input: nothing to do


@pytest.mark.parametrize("M,N,K", [(1, 64, 32), (77, 2304, 768), (128, 768, 3072), (128, 3072, 768), (33, 128, 96)])
def test_prefill_gemm_matches_float64(M, N, K):
    need_gpu()
    rng = np.random.default_rng(M * 7 + N + K)
    A = rng.standard_normal((M, K)).astype(np.float32)
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    Ad, Wd = torch.from_numpy(A).cuda(), torch.from_numpy(W).cuda()
    C = torch.full((M, N), np.nan, dtype=torch.float32, device="cuda")
    assert g.gpt2_test_gemm(Ad.data_ptr(), Wd.data_ptr(), C.data_ptr(), M, N, K, 0) == 0
    torch.cuda.synchronize()
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    bound = 2 * K * 2.0 ** -24 * (np.abs(A).astype(np.float64) @ np.abs(W).T.astype(np.float64))
    assert np.all(np.abs(C.cpu().numpy() - ref) <= bound + 1e-30)


@pytest.mark.parametrize("M,N,K,gelu", [(128, 2304, 768, 0), (128, 3072, 768, 1), (77, 2304, 768, 0), (1, 16, 64, 1),
                                        (33, 48, 128, 0)])
def test_prefill_full_k_gemm_bias_gelu(M, N, K, gelu):
    """The FC projection's kernel (all of K in 16-column tiles, bias and GELU in
    the epilogue) against float64 products; with GELU, against the oracle's GELU of
    the float64 result, within the GELU's slope times the product bound plus a few
    ulps of its own rounding."""
    need_gpu()
    rng = np.random.default_rng(M * 11 + N + K + gelu)
    A = rng.standard_normal((M, K)).astype(np.float32)
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    b = (0.1 * rng.standard_normal(N)).astype(np.float32)
    Ad, Wd, bd = (torch.from_numpy(x).cuda() for x in (A, W, b))
    C = torch.full((M, N), np.nan, dtype=torch.float32, device="cuda")
    assert g.gpt2_test_gemm_bias(Ad.data_ptr(), Wd.data_ptr(), bd.data_ptr(), C.data_ptr(), M, N, K, gelu, 0) == 0
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    lin = A.astype(np.float64) @ W.astype(np.float64).T + b.astype(np.float64)
    bound = 2 * (K + 1) * 2.0 ** -24 * (np.abs(A).astype(np.float64) @ np.abs(W).T.astype(np.float64) + np.abs(b))
    if not gelu:
        assert np.all(np.abs(got - lin) <= bound + 1e-30)
    else:
        ref = oracle.gelu(lin.astype(np.float32).ravel()).reshape(M, N).astype(np.float64)
        assert np.all(np.abs(got - ref) <= 1.2 * bound + 8 * 2.0 ** -24 * np.abs(ref) + 1e-7)


WIDTH = 768  # model width: the LayerNorm length


def _ln_rows(rng):
    """Rows that stress the workgroup evaluation of the ordered LayerNorm sums: zero
    mean (the running sum passes near 0, where its estimate is many steps off), a
    large offset, outliers, magnitudes from 1e-30 to 1e15, exact zeros, constants,
    cancelling pairs, and the residual-stream scale of the decode path."""
    n = WIDTH
    rows = [
        rng.standard_normal(n),
        0.03 * rng.standard_normal(n),
        1000.0 + rng.standard_normal(n),
        0.05 * rng.standard_normal(n) + (rng.random(n) < 0.01) * 30.0 * rng.standard_normal(n),
        rng.standard_normal(n) * 10.0 ** rng.integers(-30, 15, n),
        np.zeros(n),
        np.full(n, 0.1),
        np.repeat([1e7, -1e7], n // 2) + rng.standard_normal(n),
        np.ravel(np.column_stack([rng.standard_normal(n // 2), -rng.standard_normal(n // 2)])),
        1e-39 * rng.standard_normal(n),
    ]
    rows += [rng.standard_normal(n) * rng.uniform(0.01, 10) + rng.uniform(-1, 1) for _ in range(54)]
    return np.stack(rows).astype(np.float32)


def test_workgroup_sequential_layernorm_bit_exact():
    """The int8 path's LayerNorm, evaluated by the workgroup speculation, against the
    oracle's ordered loop: every output bit equal, on rows chosen so that the
    speculation misses (and falls back) often as well as never."""
    need_gpu()
    rng = np.random.default_rng(1234)
    x = _ln_rows(rng)
    gam = (1.0 + 0.1 * rng.standard_normal(WIDTH)).astype(np.float32)
    bet = (0.1 * rng.standard_normal(WIDTH)).astype(np.float32)
    xd, gd, bd = (torch.from_numpy(a).cuda() for a in (x, gam, bet))
    y = torch.full_like(xd, np.nan)
    assert g.gpt2_test_layernorm_seq(xd.data_ptr(), x.shape[0], gd.data_ptr(), bd.data_ptr(), y.data_ptr(), 0) == 0
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    for r in range(x.shape[0]):
        ref = oracle.layernorm(x[r].copy(), gam, bet)
        assert np.array_equal(got[r].view(np.uint32), ref.view(np.uint32)), f"row {r}"
    assert g.gpt2_test_layernorm_seq(0, 0, 0, 0, 0, 0) == 0  # no rows: nothing to do
