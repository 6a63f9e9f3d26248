"""int8 group-64 cachedStep on the GPU against the oracle (marXiv 2609.00018 abstract).

128-position session from an empty cache with the 128-step session's tokens.
- For every position and every projection (48 block projections and the head) the
  GPU records its fp32 projection input, input codes and scales, int32 group
  accumulators and output.  The oracle quantizes the captured input and
  accumulates it with its own weight codes: codes, scales, accumulators and
  outputs must be bit-identical (the abstract's captured-operand identity).
- Every fp32 operation of the int8 path (embedding, sequential-sum LayerNorm,
  attention, the specified exponential and tanh, residual adds, the fixed-order
  rescale) follows the oracle's operation order, so the 6,432,896 logits and the
  cache of the session are bit-identical to the oracle's (which implies the
  required max |diff| <= 5e-3).
"""
import numpy as np
import pytest
import torch

import oracle
import stream_gpt_transformer_amd as g
import synth
from gpu_common import D, PER, TOL_Q8, check_logits, checkpoint, model, need_gpu, oracle_q8, oracle_session

pytestmark = pytest.mark.gpu

BIAS = {0: "attn_b", 1: "attnproj_b", 2: "fc_b", 3: "mlpproj_b"}


def _views(cap: np.ndarray, layer: int, mi: int):
    o = g.gpt2_q8_capture_offsets(layer, mi)
    N = (2304, 768, 3072, 768, 50257)[mi]
    K = 3072 if mi == 3 else 768
    G = K // 64
    return dict(
        x=cap[o["in"]:o["in"] + 4 * K].view(np.float32),
        xc=cap[o["codes"]:o["codes"] + K].view(np.int8),
        xs=cap[o["scales"]:o["scales"] + 4 * G].view(np.float32),
        acc=cap[o["acc"]:o["acc"] + 4 * N * G].view(np.int32).reshape(N, G),
        y=cap[o["out"]:o["out"] + 4 * N].view(np.float32),
        N=N, K=K)


def test_q8_session_capture_bit_exact_and_logits():
    need_gpu()
    m = model()
    w = checkpoint()
    off = synth.offsets(D)
    codes, scales = oracle_q8()
    toks = synth.make_tokens(synth.SEED_SESSION, 128)
    ref, ref_cache = oracle_session(0, tuple(toks.tolist()), q8=True)
    ref_f32, _ = oracle_session(0, tuple(toks.tolist()))

    wmats = {}
    for layer in range(12):
        for mi, name in enumerate(oracle.MATRICES):
            if mi == 4 and layer:
                continue
            N, K = (2304, 768, 3072, 768, 50257)[mi], (3072 if mi == 3 else 768)
            co, so = oracle.q8_offsets(D, layer, name)
            b = None
            if mi < 4:
                o, n = off[f"h{layer}.{BIAS[mi]}"]
                b = w[o:o + n].copy()
            wmats[(layer, mi)] = (codes[co:co + N * K].reshape(N, K), scales[so:so + N * (K // 64)].reshape(N, K // 64), b)

    cap = torch.zeros(g.gpt2_q8_capture_nbytes(), dtype=torch.uint8, device="cuda")
    cache = m.new_cache(128)
    lg = torch.empty((128, g.GPT2_VOCAB), dtype=torch.float32, device="cuda")
    oracle.set_threads(16)
    n_checked = 0
    for p in range(128):
        rc = g.gpt2_q8_cached_step_capture(m.handle, cache.data_ptr(), p * PER, int(toks[p]), p, m.ws.data_ptr(),
                                           lg[p].data_ptr(), cap.data_ptr(), 0)
        assert rc == 0
        torch.cuda.synchronize()
        hc = cap.cpu().numpy()
        for (layer, mi), (wc, ws, b) in wmats.items():
            v = _views(hc, layer, mi)
            xc, xs, acc, y = oracle.q8_linear(v["x"].copy(), wc, ws, b)
            where = f"pos {p} layer {layer} matrix {mi}"
            assert np.array_equal(v["xc"], xc), where
            assert np.array_equal(v["xs"].view(np.uint32), xs.view(np.uint32)), where
            assert np.array_equal(v["acc"], acc), where
            assert np.array_equal(v["y"].view(np.uint32), y.view(np.uint32)), where
            n_checked += 1
        # the head output is the step's logits
        assert np.array_equal(_views(hc, 0, 4)["y"], lg[p].cpu().numpy())
    assert n_checked == 128 * 49
    got = lg.cpu().numpy()
    err = check_logits(got, ref, TOL_Q8, "int8 session")
    # Every fp32 step of the int8 path follows the specification's operation order,
    # so the whole session is bit-identical to the oracle: 6,432,896 logits and the
    # 128-position cache.
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(cache.cpu().numpy().view(np.uint32), ref_cache.view(np.uint32))
    print(f"int8 session: bit-identical to the oracle (max |diff| {err:.1e}); deviation from the "
          f"fp32 oracle {np.abs(got - ref_f32).max():.3f}")


def test_q8_plain_step_equals_capture_step():
    need_gpu()
    m = model()
    toks = synth.make_tokens(3, 6)
    a = m.new_cache(6)
    b = m.new_cache(6)
    la = torch.empty(g.GPT2_VOCAB, device="cuda")
    lb = torch.empty(g.GPT2_VOCAB, device="cuda")
    cap = torch.zeros(g.gpt2_q8_capture_nbytes(), dtype=torch.uint8, device="cuda")
    for p in range(6):
        m.step(a, p, int(toks[p]), la, q8=True)
        assert g.gpt2_q8_cached_step_capture(m.handle, b.data_ptr(), p * PER, int(toks[p]), p, m.ws.data_ptr(),
                                             lb.data_ptr(), cap.data_ptr(), 0) == 0
        torch.cuda.synchronize()
        assert torch.equal(la, lb)
    assert torch.equal(a, b)
