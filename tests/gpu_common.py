"""Shared set-up for the GPU tests: device buffers from torch, the packed model,
and oracle sessions computed once per test session."""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import stream_gpt_transformer_amd as g
import synth

D = synth.GPT2
PER = g.GPT2_CACHE_WORDS_PER_POS

# fp32 decode and prefill: max |logit difference| against the oracle;
# int8 path: after the fp32 rescale.
TOL_F32 = 2e-3
TOL_Q8 = 5e-3
# Greedy choices must agree wherever the oracle's top-2 gap exceeds this.
ARGMAX_GAP = 1e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@functools.lru_cache(maxsize=None)
def checkpoint(seed: int = 0, robust: bool = False, peaked: bool = False) -> np.ndarray:
    return synth.make_checkpoint(seed, D, robust=robust, peaked=peaked)


@functools.lru_cache(maxsize=None)
def model(seed: int = 0, robust: bool = False, flags: int = 3, peaked: bool = False) -> g.Model:
    ck = torch.from_numpy(checkpoint(seed, robust, peaked)).cuda()
    m = g.Model(ck, flags)
    torch.cuda.synchronize()
    del ck
    return m


@functools.lru_cache(maxsize=None)
def oracle_q8(seed: int = 0, robust: bool = False):
    return oracle.q8_quantize_weights(D, checkpoint(seed, robust))


@functools.lru_cache(maxsize=None)
def oracle_session(seed: int, toks_key: tuple, q8: bool = False, robust: bool = False):
    toks = np.array(toks_key, dtype=np.uint32)
    oracle.set_threads(16)
    return oracle.session(D, checkpoint(seed, robust), toks, q8=oracle_q8(seed, robust) if q8 else None)


@functools.lru_cache(maxsize=None)
def oracle_session_f16(seed: int, toks_key: tuple, robust: bool = False):
    toks = np.array(toks_key, dtype=np.uint32)
    oracle.set_threads(16)
    w = checkpoint(seed, robust)
    return oracle.session(D, w, toks, f16=oracle.f16_weights(D, w))


def gpu_session(m: g.Model, toks, q8: bool = False, f16: bool = False):
    """cachedStep at positions 0..T-1 from an empty cache; returns (logits [T][V], cache)."""
    T = len(toks)
    cache = m.new_cache(T)
    out = torch.empty((T, g.GPT2_VOCAB), dtype=torch.float32, device="cuda")
    for p in range(T):
        m.step(cache, p, int(toks[p]), out[p], q8=q8, f16=f16)
    torch.cuda.synchronize()
    assert m.status() == 0, f"workspace error {m.status()}"
    return out.cpu().numpy(), cache.cpu().numpy()


def check_logits(got: np.ndarray, ref: np.ndarray, tol: float, what: str = ""):
    """max |diff| <= tol and greedy agreement wherever the reference top-2 gap > ARGMAX_GAP."""
    got = np.atleast_2d(got)
    ref = np.atleast_2d(ref)
    assert np.all(np.isfinite(got)), what
    d = np.abs(got - ref).max(axis=1)
    worst = int(d.argmax())
    assert d.max() <= tol, f"{what}: max |diff| {d.max():.3e} at row {worst}"
    top2 = np.sort(ref, axis=1)[:, -2:]
    gap = top2[:, 1] - top2[:, 0]
    rows = gap > ARGMAX_GAP
    assert np.array_equal(got[rows].argmax(1), ref[rows].argmax(1)), what
    return float(d.max())
