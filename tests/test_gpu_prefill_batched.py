"""Full-prefix infer (prefill) and the batched step on the GPU.

- infer on 128 uniform-random tokens against the oracle's infer (max |diff| <= 2e-3),
  plus the edge lengths 1 and 77 (a ragged row tile).
- 64 sessions of 128 positions advanced together by the batched step: every
  session's logits and cache are bit-identical to that session run alone at
  batch 1 (batch invariance, muInference page: nondeterministic serving comes from
  reductions that change with batch shape); SHA-256 fingerprints of the logit
  streams (muInference page, fingerprint paragraph) are compared; sampled sessions
  against the oracle.
- Sessions at different positions in one batched call.
"""
import hashlib

import numpy as np
import pytest
import torch

import oracle
import stream_gpt_transformer_amd as g
import synth
from gpu_common import D, PER, TOL_F32, check_logits, checkpoint, model, need_gpu, oracle_session

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [128, 1, 77])
def test_infer_matches_oracle(n):
    need_gpu()
    toks = synth.make_tokens(synth.SEED_PREFILL, 128)[:n]
    oracle.set_threads(16)
    rc, ref = oracle.infer(D, checkpoint(), toks)
    assert rc == 0
    out = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    model().infer(toks, out)
    torch.cuda.synchronize()
    check_logits(out.cpu().numpy(), ref, TOL_F32, f"infer({n})")


def test_batched_64_sessions_bit_identical_to_batch1():
    need_gpu()
    m = model()
    B, T = 64, 128
    toks = np.stack([synth.make_tokens(synth.SEED_BATCH_BASE + s, T) for s in range(B)])
    caches = m.new_cache(T, batch=B)
    single = m.new_cache(T, batch=B)
    lb = torch.empty((B, g.GPT2_VOCAB), dtype=torch.float32, device="cuda")
    l1 = torch.empty((B, g.GPT2_VOCAB), dtype=torch.float32, device="cuda")
    hb = [hashlib.sha256() for _ in range(B)]
    h1 = [hashlib.sha256() for _ in range(B)]
    keep = {0: [], 37: []}
    for p in range(T):
        m.batched_step(caches, [p] * B, toks[:, p].tolist(), lb)
        for s in range(B):
            m.step(single[s], p, int(toks[s, p]), l1[s])
        torch.cuda.synchronize()
        assert torch.equal(lb, l1), f"position {p}"
        hbn, h1n = lb.cpu().numpy(), l1.cpu().numpy()
        for s in range(B):
            hb[s].update(hbn[s].tobytes())
            h1[s].update(h1n[s].tobytes())
        for s in keep:
            keep[s].append(hbn[s].copy())
    assert torch.equal(caches, single)
    assert [h.hexdigest() for h in hb] == [h.hexdigest() for h in h1]
    for s, rows in keep.items():
        ref, _ = oracle_session(0, tuple(toks[s].tolist()))
        check_logits(np.stack(rows), ref, TOL_F32, f"batched session {s}")


def test_batched_mixed_positions_and_batch_of_one():
    need_gpu()
    m = model()
    B = 9
    start = [0, 3, 17, 5, 100, 126, 1, 64, 9]
    toks = [synth.make_tokens(200 + s, start[s] + 2) for s in range(B)]
    caches = m.new_cache(128, batch=B)
    single = m.new_cache(128, batch=B)
    lg = torch.empty(g.GPT2_VOCAB, device="cuda")
    # bring each session to its start position with batch-1 steps
    for s in range(B):
        for p in range(start[s]):
            m.step(caches[s], p, int(toks[s][p]), lg)
    single.copy_(caches)
    lb = torch.empty((B, g.GPT2_VOCAB), device="cuda")
    l1 = torch.empty((B, g.GPT2_VOCAB), device="cuda")
    for r in range(2):
        pos = [start[s] + r for s in range(B)]
        m.batched_step(caches, pos, [int(toks[s][pos[s]]) for s in range(B)], lb)
        for s in range(B):
            m.step(single[s], pos[s], int(toks[s][pos[s]]), l1[s])
        torch.cuda.synchronize()
        assert torch.equal(lb, l1)
    assert torch.equal(caches, single)
    # B = 1 through the batched entry point equals the batch-1 entry point
    c1, c2 = m.new_cache(1), m.new_cache(1)
    a = torch.empty((1, g.GPT2_VOCAB), device="cuda")
    m.batched_step(c1.view(1, -1), [0], [123], a)
    m.step(c2, 0, 123, lg)
    torch.cuda.synchronize()
    assert torch.equal(a[0], lg) and torch.equal(c1, c2)


def test_batched_rejections():
    need_gpu()
    m = model()
    caches = m.new_cache(2, batch=2)
    lb = torch.full((2, g.GPT2_VOCAB), 7.0, device="cuda")
    h, ws, c, l, st = m.handle, m.ws.data_ptr(), caches.data_ptr(), lb.data_ptr(), caches.shape[1]
    assert g.gpt2_batched_cached_step(h, c, st, [0, 0], [1, g.GPT2_VOCAB], [0, 0], ws, l) == g.GPT2_ETOKEN
    assert g.gpt2_batched_cached_step(h, c, st, [0, PER], [1, 1], [0, 0], ws, l) == g.GPT2_ECACHE
    assert g.gpt2_batched_cached_step(h, c, st, [0, 2 * PER], [1, 1], [0, 2], ws, l) == g.GPT2_ECACHE  # stride too short
    assert g.gpt2_batched_cached_step(h, c, st, [0, 0], [1, 1], [0, 128], ws, l) == g.GPT2_EPOSITION
    assert g.gpt2_batched_cached_step(h, c, st, [], [], [], ws, l) == g.GPT2_EARG
    assert g.gpt2_batched_cached_step(h, c, st, [0] * 65, [0] * 65, [0] * 65, ws, l) == g.GPT2_EARG
    torch.cuda.synchronize()
    assert torch.all(lb == 7.0) and torch.all(caches == 0)


def test_prefill_hands_the_session_to_the_cached_step():
    """gpt2_prefill over the first 64 tokens of the 128-token session, then
    cachedStep at positions 64..127: logits against the oracle's cached session at
    every continued position (fp32 tolerance); the handed-over cache rows against
    the oracle's; the prefill logits against the oracle's at position 63."""
    need_gpu()
    m = model()
    T, P = 128, 64
    toks = synth.make_tokens(synth.SEED_SESSION, T)
    ref, ref_cache = oracle_session(0, tuple(int(t) for t in toks))
    cache = m.new_cache(T)
    lg = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    m.prefill(toks[:P], cache, lg)
    torch.cuda.synchronize()
    check_logits(lg.cpu().numpy(), ref[P - 1], TOL_F32, "prefill logits")
    got = cache.cpu().numpy()[:P * PER]
    assert np.abs(got - ref_cache[:P * PER]).max() <= 1e-3
    out = torch.empty((T - P, g.GPT2_VOCAB), dtype=torch.float32, device="cuda")
    for p in range(P, T):
        m.step(cache, p, int(toks[p]), out[p - P])
    torch.cuda.synchronize()
    check_logits(out.cpu().numpy(), ref[P:], TOL_F32, "steps after prefill")


def test_prefill_validation():
    need_gpu()
    m = model()
    cache = m.new_cache(8)
    lg = torch.empty(g.GPT2_VOCAB, dtype=torch.float32, device="cuda")
    cap = cache.numel()
    assert g.gpt2_prefill(m.handle, [1] * 9, cache.data_ptr(), cap, m.ws.data_ptr(), lg.data_ptr()) == g.GPT2_ECACHE
    assert g.gpt2_prefill(m.handle, [], cache.data_ptr(), cap, m.ws.data_ptr(), lg.data_ptr()) == g.GPT2_ETOKEN
    assert g.gpt2_prefill(m.handle, [g.GPT2_VOCAB], cache.data_ptr(), cap, m.ws.data_ptr(), lg.data_ptr()) == g.GPT2_ETOKEN
    assert g.gpt2_prefill(m.handle, [1], 0, cap, m.ws.data_ptr(), lg.data_ptr()) == g.GPT2_ECACHE
