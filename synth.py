"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and places them in the packed checkpoint
layout; it holds none of the model's arithmetic.  Both sides of every parity
check receive the arrays built here and nothing else.

Checkpoint layout (LeanExe GPT-2 README, "packed checkpoint" paragraph): token
embeddings, all 1,024 stored position rows, twelve blocks, final normalisation,
every word little-endian binary32, 124,439,808 words in total.  The order of the
tensors inside a block is not printed on that page; this module takes GPT-2's own
parameter order with block matrices stored [input][output] (the gpt2.s page,
"weight tiling" paragraph, states that orientation for the checkpoint):

    ln1_g, ln1_b, attn_w [D][3D] (q|k|v columns), attn_b, attnproj_w [D][D],
    attnproj_b, ln2_g, ln2_b, fc_w [D][F], fc_b, mlpproj_w [F][D], mlpproj_b

Weight recipe (one seeded normal draw per embedding/matrix tensor, in checkpoint
order): N(0, 0.02) for wte, wpe and the four block matrices; LayerNorm gamma = 1,
beta = 0 and every bias 0 in the plain recipe.  The "robust" recipe also draws
biases ~ N(0, 0.02), gamma ~ 1 + N(0, 0.1) and beta ~ N(0, 0.02) so that offset
mistakes hidden by zeros and ones surface.

The "peaked" recipe takes the plain draw and multiplies the query and key columns
of every block's attn_w by PEAK_QK_SCALE (10), so attention scores spread over
tens of units instead of N(0, 0.3^2): softmax weights are close to one-hot and the
exponential's argument falls below -87 (where it underflows to 0) for most keys.
It also copies position row 5 into rows 9 and 17, so a token repeated at
positions 5, 9 and 17 gives identical layer-0 keys there (tied scores).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Dims:
    n_layer: int = 12
    d_model: int = 768
    n_head: int = 12
    d_ff: int = 3072
    vocab: int = 50257
    n_pos_rows: int = 1024   # position rows stored in the checkpoint
    max_pos: int = 128       # positions accepted by the entry points (0..127)

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_head


GPT2 = Dims()
# Small shapes for brute-force oracle checks (head_dim a power of two).
TINY = Dims(n_layer=2, d_model=64, n_head=4, d_ff=256, vocab=97, n_pos_rows=40, max_pos=32)


def block_tensors(d: Dims) -> List[Tuple[str, int, str]]:
    """(name, words, kind) for one block, in checkpoint order; kind in {gamma, beta, bias, matrix}."""
    D, F = d.d_model, d.d_ff
    return [
        ("ln1_g", D, "gamma"), ("ln1_b", D, "beta"),
        ("attn_w", D * 3 * D, "matrix"), ("attn_b", 3 * D, "bias"),
        ("attnproj_w", D * D, "matrix"), ("attnproj_b", D, "bias"),
        ("ln2_g", D, "gamma"), ("ln2_b", D, "beta"),
        ("fc_w", D * F, "matrix"), ("fc_b", F, "bias"),
        ("mlpproj_w", F * D, "matrix"), ("mlpproj_b", D, "bias"),
    ]


def layout(d: Dims = GPT2) -> List[Tuple[str, int, int, str]]:
    """Every tensor of the packed checkpoint as (name, word offset, words, kind)."""
    out: List[Tuple[str, int, int, str]] = []
    off = 0

    def put(name: str, n: int, kind: str) -> None:
        nonlocal off
        out.append((name, off, n, kind))
        off += n

    put("wte", d.vocab * d.d_model, "matrix")
    put("wpe", d.n_pos_rows * d.d_model, "matrix")
    for l in range(d.n_layer):
        for name, n, kind in block_tensors(d):
            put(f"h{l}.{name}", n, kind)
    put("lnf_g", d.d_model, "gamma")
    put("lnf_b", d.d_model, "beta")
    return out


def ckpt_words(d: Dims = GPT2) -> int:
    name, off, n, _ = layout(d)[-1]
    return off + n


def offsets(d: Dims = GPT2) -> Dict[str, Tuple[int, int]]:
    return {name: (off, n) for name, off, n, _ in layout(d)}


PEAK_QK_SCALE = 10.0
PEAK_TIED_POSITIONS = (5, 9, 17)


def make_checkpoint(seed: int = 0, d: Dims = GPT2, robust: bool = False, peaked: bool = False) -> np.ndarray:
    """Packed little-endian float32 checkpoint (numpy float32 is little-endian here)."""
    if peaked:
        w = make_checkpoint(seed, d, robust)
        offs = offsets(d)
        D = d.d_model
        for l in range(d.n_layer):
            off, n = offs[f"h{l}.attn_w"]
            m = w[off:off + n].reshape(D, 3 * D)  # [input][q | k | v]
            m[:, :2 * D] *= np.float32(PEAK_QK_SCALE)
        wpe_off, _ = offs["wpe"]
        p0 = PEAK_TIED_POSITIONS[0]
        for p in PEAK_TIED_POSITIONS[1:]:
            w[wpe_off + p * D:wpe_off + (p + 1) * D] = w[wpe_off + p0 * D:wpe_off + (p0 + 1) * D]
        return w
    rng = np.random.default_rng(seed)
    w = np.empty(ckpt_words(d), dtype="<f4")
    for name, off, n, kind in layout(d):
        dst = w[off:off + n]
        if kind == "matrix":
            dst[:] = (rng.standard_normal(n) * 0.02).astype(np.float32)
        elif kind == "gamma":
            dst[:] = 1.0 if not robust else (1.0 + rng.standard_normal(n) * 0.1).astype(np.float32)
        elif kind == "beta" or kind == "bias":
            dst[:] = 0.0 if not robust else (rng.standard_normal(n) * 0.02).astype(np.float32)
        else:  # pragma: no cover
            raise ValueError(kind)
    return w


def make_tokens(seed: int, count: int, d: Dims = GPT2) -> np.ndarray:
    """Uniform-random token ids in [0, vocab) as little-endian uint32."""
    return np.random.default_rng(seed).integers(0, d.vocab, size=count, dtype=np.uint32)


def make_tied_tokens(seed: int, count: int, d: Dims = GPT2) -> np.ndarray:
    """make_tokens with the token at the first tied position repeated at the others
    (with the peaked recipe's equal position rows, their layer-0 keys are equal)."""
    t = make_tokens(seed, count, d)
    for p in PEAK_TIED_POSITIONS[1:]:
        if p < count:
            t[p] = t[PEAK_TIED_POSITIONS[0]]
    return t


# Token seeds of the workloads: the 8-step session, the 128-step sessions (fp32 and
# int8 use the same tokens), the 128-token prefill and the 64 batched sessions.
SEED_SHORT = 100
SEED_SESSION = 101
SEED_PREFILL = 102
SEED_BATCH_BASE = 1000
SEED_PEAKED = 103
