"""ctypes wrapper of the CPU oracle (oracle/gpt2_oracle.cpp) — TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the bench's CPU-baseline leg import this
package.  The GPU library never does, and nothing here is shared with it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "gpt2_oracle.cpp")
LIB = os.path.join(_HERE, "liboracle.so")

# Plain IEEE binary32: no contraction into FMA, no fast-math, SSE arithmetic.
CXXFLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
            "-fopenmp"]


def build(verbose: bool = False) -> str:
    cmd = ["g++", *CXXFLAGS, SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


class OracleDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layer", "d_model", "n_head", "d_ff", "vocab", "n_pos_rows", "max_pos")]


_lib: Optional[ctypes.CDLL] = None

_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_i8p = np.ctypeslib.ndpointer(np.int8, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
_sz = ctypes.c_size_t
_dp = ctypes.POINTER(OracleDims)


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    L = ctypes.CDLL(LIB)
    sig = {
        "oracle_set_threads": (None, [ctypes.c_int]),
        "oracle_max_threads": (ctypes.c_int, []),
        "oracle_ckpt_words": (_sz, [_dp]),
        "oracle_cache_words_per_pos": (_sz, [_dp]),
        "oracle_tensor_offset": (ctypes.c_longlong, [_dp, ctypes.c_int, ctypes.c_int]),
        "oracle_cached_step": (ctypes.c_int, [_dp, _f32p, _sz, _f32p, _sz, ctypes.c_uint32,
                                              ctypes.c_int32, _f32p]),
        "oracle_infer": (ctypes.c_int, [_dp, _f32p, _sz, _u32p, ctypes.c_int, _f32p]),
        "oracle_q8_sizes": (None, [_dp, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
        "oracle_q8_offsets": (None, [_dp, ctypes.c_int, ctypes.c_int, ctypes.POINTER(_sz),
                                     ctypes.POINTER(_sz)]),
        "oracle_q8_quantize_weights": (ctypes.c_int, [_dp, _f32p, _sz, _i8p, _f32p]),
        "oracle_q8_cached_step": (ctypes.c_int, [_dp, _f32p, _sz, _i8p, _f32p, _f32p, _sz,
                                                 ctypes.c_uint32, ctypes.c_int32, _f32p]),
        "oracle_f16_weights": (ctypes.c_int, [_dp, _f32p, _sz, _f32p]),
        "oracle_f16_cached_step": (ctypes.c_int, [_dp, _f32p, _f32p, _sz, _f32p, _sz, ctypes.c_uint32,
                                                  ctypes.c_int32, _f32p]),
        "oracle_round_binary16": (None, [ctypes.c_longlong, _f32p, _f32p]),
        "oracle_qv_sizes": (ctypes.c_int, [_dp, ctypes.c_int, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
        "oracle_qv_quantize_weights": (ctypes.c_int, [_dp, _f32p, _sz, ctypes.c_int, _i8p, _f32p]),
        "oracle_qv_cached_step": (ctypes.c_int, [_dp, _f32p, _sz, ctypes.c_int, ctypes.c_int, _i8p, _f32p,
                                                 _f32p, _sz, ctypes.c_uint32, ctypes.c_int32, _f32p]),
        "oracle_qv_linear": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _f32p, ctypes.c_int, _i8p, _f32p,
                                            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, _f32p]),
        "oracle_layernorm": (None, [ctypes.c_int, _f32p, _f32p, _f32p, _f32p]),
        "oracle_linear": (None, [ctypes.c_int, ctypes.c_int, _f32p, _f32p, ctypes.c_void_p, _f32p]),
        "oracle_gelu": (None, [ctypes.c_int, _f32p, _f32p]),
        "oracle_special": (None, [ctypes.c_int, ctypes.c_longlong, _f32p, _f32p]),
        "oracle_special_bits": (None, [ctypes.c_int, ctypes.c_uint32, ctypes.c_longlong, _f32p]),
        "oracle_attention_head": (None, [ctypes.c_int, _f32p, _f32p, _f32p, ctypes.c_int,
                                         ctypes.c_int, _f32p, _f32p]),
        "oracle_quantize": (ctypes.c_int, [ctypes.c_int, _f32p, _i8p, _f32p]),
        "oracle_quantize_with_scale": (None, [ctypes.c_int, _f32p, ctypes.c_float, _i8p]),
        "oracle_q8_linear": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _f32p, _i8p, _f32p,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, _f32p]),
        "oracle_q8_linear_codes": (None, [ctypes.c_int, ctypes.c_int, _i8p, _f32p, _i8p, _f32p,
                                          ctypes.c_void_p, ctypes.c_void_p, _f32p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def dims(d) -> OracleDims:
    """OracleDims from any object with the synth.Dims field names."""
    return OracleDims(d.n_layer, d.d_model, d.n_head, d.d_ff, d.vocab, d.n_pos_rows, d.max_pos)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def ckpt_words(d) -> int:
    return int(lib().oracle_ckpt_words(ctypes.byref(dims(d))))


def cache_words_per_pos(d) -> int:
    return int(lib().oracle_cache_words_per_pos(ctypes.byref(dims(d))))


BLOCK_TENSORS = ["ln1_g", "ln1_b", "attn_w", "attn_b", "attnproj_w", "attnproj_b",
                 "ln2_g", "ln2_b", "fc_w", "fc_b", "mlpproj_w", "mlpproj_b"]


def tensor_offset(d, name: str, layer: int = 0) -> int:
    special = {"wte": 100, "wpe": 101, "lnf_g": 102, "lnf_b": 103}
    t = special[name] if name in special else BLOCK_TENSORS.index(name)
    return int(lib().oracle_tensor_offset(ctypes.byref(dims(d)), layer, t))


def cached_step(d, w: np.ndarray, cache: np.ndarray, cache_words: int, tok: int, pos: int
                ) -> Tuple[int, np.ndarray]:
    """cache: float32 array with room for (pos+1) positions; the first cache_words are the input."""
    logits = np.zeros(d.vocab, np.float32)
    rc = lib().oracle_cached_step(ctypes.byref(dims(d)), w, w.size, cache, cache_words,
                                  int(tok), int(pos), logits)
    return rc, logits


def infer(d, w: np.ndarray, toks: np.ndarray) -> Tuple[int, np.ndarray]:
    logits = np.zeros(d.vocab, np.float32)
    toks = np.ascontiguousarray(toks, dtype=np.uint32)
    rc = lib().oracle_infer(ctypes.byref(dims(d)), w, w.size, toks, int(toks.size), logits)
    return rc, logits


def session(d, w: np.ndarray, toks: np.ndarray, q8: Optional[Tuple[np.ndarray, np.ndarray]] = None,
            f16: Optional[np.ndarray] = None):
    """Run cachedStep at positions 0..len(toks)-1 from an empty cache (int8 with
    q8 = (codes, scales), binary16 storage with f16 = f16_weights(d, w)).
    Returns (logits [T][V], cache)."""
    T = len(toks)
    per = cache_words_per_pos(d)
    cache = np.zeros(T * per, np.float32)
    out = np.zeros((T, d.vocab), np.float32)
    for p in range(T):
        if q8 is not None:
            rc, lg = q8_cached_step(d, w, q8[0], q8[1], cache, p * per, int(toks[p]), p)
        elif f16 is not None:
            rc, lg = f16_cached_step(d, w, f16, cache, p * per, int(toks[p]), p)
        else:
            rc, lg = cached_step(d, w, cache, p * per, int(toks[p]), p)
        assert rc == 0, rc
        out[p] = lg
    return out, cache


def round_binary16(x: np.ndarray) -> np.ndarray:
    """IEEE binary16 rounding (nearest, ties to even) of float32 values, as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    lib().oracle_round_binary16(x.size, x, y)
    return y


def f16_weights(d, w: np.ndarray) -> np.ndarray:
    """Checkpoint copy with the block matrices and the token table (as the head)
    rounded to binary16."""
    w16 = np.empty_like(w)
    rc = lib().oracle_f16_weights(ctypes.byref(dims(d)), w, w.size, w16)
    assert rc == 0, rc
    return w16


def f16_cached_step(d, w, w16, cache, cache_words, tok, pos) -> Tuple[int, np.ndarray]:
    logits = np.zeros(d.vocab, np.float32)
    rc = lib().oracle_f16_cached_step(ctypes.byref(dims(d)), w, w16, w.size, cache, cache_words,
                                      int(tok), int(pos), logits)
    return rc, logits


# ---- quantizer granularity variants: weight groups gw, input groups gx (0 = whole row)

def qv_sizes(d, gw: int) -> Tuple[int, int]:
    c, s = _sz(), _sz()
    rc = lib().oracle_qv_sizes(ctypes.byref(dims(d)), gw, ctypes.byref(c), ctypes.byref(s))
    assert rc == 0, rc
    return int(c.value), int(s.value)


def qv_quantize_weights(d, w: np.ndarray, gw: int) -> Tuple[np.ndarray, np.ndarray]:
    nc, ns = qv_sizes(d, gw)
    codes = np.zeros(nc, np.int8)
    scales = np.zeros(ns, np.float32)
    rc = lib().oracle_qv_quantize_weights(ctypes.byref(dims(d)), w, w.size, gw, codes, scales)
    assert rc == 0, rc
    return codes, scales


def qv_cached_step(d, w, gw, gx, codes, scales, cache, cache_words, tok, pos) -> Tuple[int, np.ndarray]:
    logits = np.zeros(d.vocab, np.float32)
    rc = lib().oracle_qv_cached_step(ctypes.byref(dims(d)), w, w.size, gw, gx, codes, scales, cache,
                                     cache_words, int(tok), int(pos), logits)
    return rc, logits


def qv_session(d, w, toks, gw: int, gx: int, q=None):
    """Variant cachedStep at positions 0..T-1 from an empty cache; q = qv_quantize_weights(d, w, gw)."""
    codes, scales = q if q is not None else qv_quantize_weights(d, w, gw)
    T = len(toks)
    per = cache_words_per_pos(d)
    cache = np.zeros(T * per, np.float32)
    out = np.zeros((T, d.vocab), np.float32)
    for p in range(T):
        rc, out[p] = qv_cached_step(d, w, gw, gx, codes, scales, cache, p * per, int(toks[p]), p)
        assert rc == 0, rc
    return out, cache


def qv_linear(x, gx: int, wc, ws, gw: int, b=None):
    """Returns (codes, input scales, accumulators [N][K/gcd], y) of one variant projection."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    wc = np.ascontiguousarray(wc, dtype=np.int8)
    ws = np.ascontiguousarray(ws, dtype=np.float32)
    N, K = wc.shape
    GX = K if gx == 0 else gx
    GW = K if gw == 0 else gw
    import math
    GM = math.gcd(GX, GW)
    xc = np.zeros(K, np.int8)
    xs = np.zeros(K // GX, np.float32)
    acc = np.zeros((N, K // GM), np.int32)
    y = np.zeros(N, np.float32)
    bb = None if b is None else np.ascontiguousarray(b, dtype=np.float32)
    rc = lib().oracle_qv_linear(K, N, x, gx, wc, ws, gw, None if bb is None else bb.ctypes.data,
                                xc.ctypes.data, xs.ctypes.data, acc.ctypes.data, y)
    assert rc == 0, rc
    return xc, xs, acc, y


def q8_sizes(d) -> Tuple[int, int]:
    c, s = _sz(), _sz()
    lib().oracle_q8_sizes(ctypes.byref(dims(d)), ctypes.byref(c), ctypes.byref(s))
    return int(c.value), int(s.value)


MATRICES = ["attn_w", "attnproj_w", "fc_w", "mlpproj_w", "head"]


def q8_offsets(d, layer: int, matrix: str) -> Tuple[int, int]:
    c, s = _sz(), _sz()
    lib().oracle_q8_offsets(ctypes.byref(dims(d)), layer, MATRICES.index(matrix),
                            ctypes.byref(c), ctypes.byref(s))
    return int(c.value), int(s.value)


def q8_quantize_weights(d, w: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    nc, ns = q8_sizes(d)
    codes = np.zeros(nc, np.int8)
    scales = np.zeros(ns, np.float32)
    rc = lib().oracle_q8_quantize_weights(ctypes.byref(dims(d)), w, w.size, codes, scales)
    assert rc == 0, rc
    return codes, scales


def q8_cached_step(d, w, codes, scales, cache, cache_words, tok, pos) -> Tuple[int, np.ndarray]:
    logits = np.zeros(d.vocab, np.float32)
    rc = lib().oracle_q8_cached_step(ctypes.byref(dims(d)), w, w.size, codes, scales, cache,
                                     cache_words, int(tok), int(pos), logits)
    return rc, logits


def layernorm(x, g, b) -> np.ndarray:
    y = np.zeros_like(x)
    lib().oracle_layernorm(x.size, x, g, b, y)
    return y


def linear(x, W_in_out, b=None) -> np.ndarray:
    K, N = W_in_out.shape
    y = np.zeros(N, np.float32)
    lib().oracle_linear(K, N, x, np.ascontiguousarray(W_in_out), _ptr(b), y)
    return y


def gelu(x) -> np.ndarray:
    y = np.zeros_like(x)
    lib().oracle_gelu(x.size, x, y)
    return y


def exp_spec(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.zeros_like(x)
    lib().oracle_special(0, x.size, x, y)
    return y


def tanh_spec(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.zeros_like(x)
    lib().oracle_special(1, x.size, x, y)
    return y


def special_bits(kind: int, first: int, n: int) -> np.ndarray:
    """f(x) for every binary32 bit pattern first..first+n-1 (kind 0 exp, 1 tanh)."""
    y = np.zeros(n, np.float32)
    lib().oracle_special_bits(kind, first, n, y)
    return y


def attention_head(q, K, V) -> Tuple[np.ndarray, np.ndarray]:
    """q [dh]; K, V [npos][dh] -> (a [dh], softmax weights [npos])."""
    npos, dh = K.shape
    a = np.zeros(dh, np.float32)
    wts = np.zeros(npos, np.float32)
    lib().oracle_attention_head(dh, q, np.ascontiguousarray(K), np.ascontiguousarray(V), dh, npos,
                                a, wts)
    return a, wts


def quantize(x) -> Tuple[np.ndarray, np.ndarray]:
    codes = np.zeros(x.size, np.int8)
    scales = np.zeros(x.size // 64, np.float32)
    rc = lib().oracle_quantize(x.size, x, codes, scales)
    assert rc == 0, rc
    return codes, scales


def quantize_with_scale(x, s: float) -> np.ndarray:
    codes = np.zeros(x.size, np.int8)
    lib().oracle_quantize_with_scale(x.size, x, ctypes.c_float(s), codes)
    return codes


def q8_linear(x, wc, ws, b=None):
    """x [K] fp32; wc [N][K] int8; ws [N][K/64] -> (xc, xs, acc [N][G], y)."""
    N, K = wc.shape
    xc = np.zeros(K, np.int8)
    xs = np.zeros(K // 64, np.float32)
    acc = np.zeros((N, K // 64), np.int32)
    y = np.zeros(N, np.float32)
    rc = lib().oracle_q8_linear(K, N, x, np.ascontiguousarray(wc), np.ascontiguousarray(ws),
                                _ptr(b), _ptr(xc), _ptr(xs), _ptr(acc), y)
    assert rc == 0, rc
    return xc, xs, acc, y


def q8_linear_codes(xc, xs, wc, ws, b=None):
    N, K = wc.shape
    acc = np.zeros((N, K // 64), np.int32)
    y = np.zeros(N, np.float32)
    lib().oracle_q8_linear_codes(K, N, xc, xs, np.ascontiguousarray(wc), np.ascontiguousarray(ws),
                                 _ptr(b), _ptr(acc), y)
    return acc, y
