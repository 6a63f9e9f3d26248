"""fp32 cachedStep and infer on the GPU against the oracle.

- 8-step session from an empty cache (positions 0..7), logits compared every step.
- 128-step session (positions 0..127); every position cross-checked against the
  GPU full-prefix infer over the same prefix and against the oracle (whose infer
  equals its cached chain bit for bit).
- Random biases/gamma/beta, so offset mistakes hidden by zeros surface.
- Caches against the oracle's; determinism; host-side rejections with a real model.
Tolerance: max |logit difference| <= 2e-3; greedy choices agree wherever the
oracle's top-2 gap exceeds 1e-2.
"""
import hashlib

import numpy as np
import pytest
import torch

import stream_gpt_transformer_amd as g
import synth
from gpu_common import (D, PER, TOL_F32, check_logits, gpu_session, model, need_gpu, oracle_session)

pytestmark = pytest.mark.gpu


def test_short_session_positions_0_to_7():
    need_gpu()
    toks = synth.make_tokens(synth.SEED_SHORT, 8)
    ref, ref_cache = oracle_session(0, tuple(toks.tolist()))
    got, cache = gpu_session(model(), toks)
    check_logits(got, ref, TOL_F32, "8-step session")
    assert np.abs(cache[:8 * PER] - ref_cache).max() <= 1e-4


def test_full_session_128_positions_and_infer_cross_check():
    need_gpu()
    toks = synth.make_tokens(synth.SEED_SESSION, 128)
    ref, ref_cache = oracle_session(0, tuple(toks.tolist()))
    m = model()
    got, cache = gpu_session(m, toks)
    check_logits(got, ref, TOL_F32, "128-step session")
    assert np.abs(cache - ref_cache).max() <= 1e-4
    # full-prefix infer at every prefix length, GPU against GPU cached and oracle
    out = torch.empty((128, g.GPT2_VOCAB), dtype=torch.float32, device="cuda")
    for t in range(128):
        m.infer(toks[:t + 1], out[t])
    torch.cuda.synchronize()
    inf = out.cpu().numpy()
    check_logits(inf, ref, TOL_F32, "infer vs oracle")
    assert np.abs(inf - got).max() <= TOL_F32


def test_robust_weights_session():
    need_gpu()
    toks = synth.make_tokens(7, 24)
    ref, ref_cache = oracle_session(1, tuple(toks.tolist()), robust=True)
    got, cache = gpu_session(model(1, True, 1), toks)
    check_logits(got, ref, TOL_F32, "robust weights")
    assert np.abs(cache[:24 * PER] - ref_cache).max() <= 1e-4


@pytest.mark.parametrize("q8", [False, True], ids=["fp32", "int8"])
def test_fused_step_equals_phase_kernels(q8):
    """The single-launch step and the one-kernel-per-phase path compute the same bits
    (logits and caches) over a 40-position session; the workspace reports no error."""
    need_gpu()
    m = model()
    toks = synth.make_tokens(21, 40)
    fused, cf = gpu_session(m, toks, q8=q8)
    assert m.status() == 0
    g.gpt2_test_force_phase_kernels(True)
    try:
        phase, cp = gpu_session(m, toks, q8=q8)
    finally:
        g.gpt2_test_force_phase_kernels(False)
    assert np.array_equal(fused.view(np.uint32), phase.view(np.uint32))
    assert np.array_equal(cf.view(np.uint32), cp.view(np.uint32))


def test_deterministic_bits():
    need_gpu()
    toks = synth.make_tokens(5, 16)
    m = model()
    a, ca = gpu_session(m, toks)
    b, cb = gpu_session(m, toks)
    assert hashlib.sha256(a.tobytes()).digest() == hashlib.sha256(b.tobytes()).digest()
    assert np.array_equal(ca, cb)


def test_step_uses_supplied_cache_contents():
    """A step at position p reads the prior rows as supplied: a perturbed row changes
    the logits; restoring it restores them bit for bit."""
    need_gpu()
    m = model()
    toks = synth.make_tokens(9, 6)
    cache = m.new_cache(6)
    lg = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    for p in range(5):
        m.step(cache, p, int(toks[p]), lg)
    saved = cache.clone()
    m.step(cache, 5, int(toks[5]), lg)
    base = lg.clone()
    cache.copy_(saved)
    cache[PER + 100] += 1.0
    m.step(cache, 5, int(toks[5]), lg)
    assert not torch.equal(lg, base)
    cache.copy_(saved)
    m.step(cache, 5, int(toks[5]), lg)
    assert torch.equal(lg, base)


def test_rejections_leave_outputs_untouched():
    need_gpu()
    m = model()
    cache = m.new_cache(4)
    lg = torch.full((g.GPT2_VOCAB,), 7.0, device="cuda")
    h, ws, c, l = m.handle, m.ws.data_ptr(), cache.data_ptr(), lg.data_ptr()
    assert g.gpt2_cached_step(h, c, 0, g.GPT2_VOCAB, 0, ws, l) == g.GPT2_ETOKEN
    assert g.gpt2_cached_step(h, c, 0, -1, 0, ws, l) == g.GPT2_ETOKEN
    assert g.gpt2_cached_step(h, c, 128 * PER, 0, 128, ws, l) == g.GPT2_EPOSITION
    assert g.gpt2_cached_step(h, c, 0, 0, -1, ws, l) == g.GPT2_EPOSITION
    assert g.gpt2_cached_step(h, c, PER, 0, 0, ws, l) == g.GPT2_ECACHE
    assert g.gpt2_cached_step(h, c, 0, 0, 1, ws, l) == g.GPT2_ECACHE
    assert g.gpt2_cached_step(h, 0, 0, 0, 0, ws, l) == g.GPT2_ECACHE
    assert g.gpt2_cached_step(h, c, 0, 0, 0, 0, l) == g.GPT2_EARG
    assert g.gpt2_infer(h, [], ws, l) == g.GPT2_ETOKEN
    assert g.gpt2_infer(h, [0] * 129, ws, l) == g.GPT2_ETOKEN
    assert g.gpt2_infer(h, [0, g.GPT2_VOCAB], ws, l) == g.GPT2_ETOKEN
    mf = model(1, True, 1)  # fp32-only model
    assert g.gpt2_q8_cached_step(mf.handle, c, 0, 0, 0, ws, l) == g.GPT2_ENOTPACKED
    torch.cuda.synchronize()
    assert torch.all(lg == 7.0) and torch.all(cache == 0)


@pytest.mark.parametrize("q8,f16", [(False, False), (True, False), (False, True)], ids=["fp32", "int8", "binary16"])
def test_timestamp_hook_changes_no_bits_and_orders_phases(q8, f16):
    """With the single-launch step's timestamp hook on, a session computes the same bits.
    Every workgroup stamps its start, head input, head rows done and end in that order;
    the units of the set that computes block l stamp that block's phase inputs in causal
    order (regular units: x in, own QKV rows published, x1 in, GELU slice in; head
    units: reduce-scatter share, attention output, x1 published), and no unit stamps a
    block of the other set.  Turned off, the hook writes nothing."""
    need_gpu()
    m = model(flags=g.GPT2_PACK_F32 | g.GPT2_PACK_Q8 | g.GPT2_PACK_F16) if f16 else model()
    toks = synth.make_tokens(23, 6)
    ref, cref = gpu_session(m, toks, q8=q8, f16=f16)
    trace = torch.zeros(256 * 64, dtype=torch.int64, device="cuda")
    g.gpt2_test_fused_trace(trace.data_ptr())
    try:
        got, cgot = gpu_session(m, toks, q8=q8, f16=f16)  # the trace holds the last step's stamps
    finally:
        g.gpt2_test_fused_trace(None)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(cgot.view(np.uint32), cref.view(np.uint32))
    tr = trace.view(256, 64).cpu().numpy()
    for b in range(256):
        X, rank = b % 8, b // 8
        st, q = rank % 2, rank // 2
        head = q < (2 if X < 4 else 1)
        t = tr[b]
        assert 0 < t[0] <= t[49] <= t[55] <= t[50] <= t[51], (b, t[[0, 49, 55, 50, 51]])
        slots = (1, 2, 3) if head else (1, 2, 3, 4)
        prev = t[0]
        for l in range(12):
            s = [t[k + 4 * l] for k in slots]
            if l % 2 != st:
                assert all(v == 0 for v in s), (b, l, s)
                continue
            assert prev <= s[0] and all(s[i] <= s[i + 1] for i in range(len(s) - 1)), (b, l, prev, s)
            prev = s[-1]
        assert prev <= t[49]
    # off: a later step leaves the buffer untouched
    trace.zero_()
    cache = m.new_cache(1)
    lg = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    m.step(cache, 0, int(toks[0]), lg, q8=q8, f16=f16)
    torch.cuda.synchronize()
    assert int(trace.abs().sum().item()) == 0
    assert m.status() == 0
