"""Python binding of libgpt2mi.so (GPT-2 124M cached decode on MI355X).

The functions named gpt2_* mirror the C-ABI in include/gpt2.h one to one and only
marshal arguments: every step of the computation runs in the HIP kernels of the
library.  Device memory and streams come from torch (plumbing only): pass
`tensor.data_ptr()` for device pointers and `torch.cuda.current_stream().cuda_stream`
(or 0) for streams.  There is no CPU fallback: if the library is missing this
module raises on first use.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgpt2mi.so")

GPT2_LAYERS = 12
GPT2_DMODEL = 768
GPT2_HEADS = 12
GPT2_DFF = 3072
GPT2_VOCAB = 50257
GPT2_MAX_POS = 128
GPT2_CKPT_WORDS = 124_439_808
GPT2_CKPT_BYTES = 497_759_232
GPT2_CACHE_WORDS_PER_POS = 18_432
GPT2_MAX_BATCH = 64
GPT2_NOALLOC_SCRATCH_BYTES = 6_555_904
GPT2_PACK_F32 = 1
GPT2_PACK_Q8 = 2
GPT2_PACK_F16 = 4
GPT2_WEIGHTS_F32, GPT2_WEIGHTS_Q8, GPT2_WEIGHTS_F16 = 0, 1, 2
GPT2_OK, GPT2_EWEIGHTS, GPT2_ETOKEN, GPT2_EPOSITION, GPT2_ECACHE, GPT2_ENOTPACKED, GPT2_EARG, GPT2_EHIP = \
    0, -1, -2, -3, -4, -5, -6, -7
ERROR_NAMES = {0: "GPT2_OK", -1: "GPT2_EWEIGHTS", -2: "GPT2_ETOKEN", -3: "GPT2_EPOSITION",
               -4: "GPT2_ECACHE", -5: "GPT2_ENOTPACKED", -6: "GPT2_EARG", -7: "GPT2_EHIP"}

# Every symbol include/gpt2.h declares, with (restype, argtypes).
_vp, _sz, _i, _u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32
SIGNATURES = {
    "gpt2_packed_nbytes": (_sz, [_i]),
    "gpt2_workspace_nbytes": (_sz, []),
    "gpt2_pack_weights": (_i, [_vp, _sz, _vp, _sz, _i, _vp, ctypes.POINTER(_vp)]),
    "gpt2_release": (None, [_vp]),
    "gpt2_cached_step": (_i, [_vp, _vp, _sz, _u32, ctypes.c_int32, _vp, _vp, _vp]),
    "gpt2_q8_cached_step": (_i, [_vp, _vp, _sz, _u32, ctypes.c_int32, _vp, _vp, _vp]),
    "gpt2_f16_cached_step": (_i, [_vp, _vp, _sz, _u32, ctypes.c_int32, _vp, _vp, _vp]),
    "gpt2_q8_cached_step_grouped": (_i, [_vp, _i, _vp, _sz, _u32, ctypes.c_int32, _vp, _vp, _vp]),
    "gpt2_pack_weights_grouped": (_i, [_vp, _sz, _vp, _sz, _i, _i, _vp, ctypes.POINTER(_vp)]),
    "gpt2_q8_weight_group": (_i, [_vp]),
    "gpt2_batched_cached_step": (_i, [_vp, _vp, _sz, _vp, _vp, _vp, _i, _vp, _vp, _vp]),
    "gpt2_cached_step_noalloc": (_i, [_vp, _vp, _sz, _u32, ctypes.c_int32, _vp, _vp, _vp]),
    "gpt2_infer": (_i, [_vp, _vp, _i, _vp, _vp, _vp]),
    "gpt2_generate": (_i, [_vp, _vp, _sz, _vp, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "gpt2_prefill": (_i, [_vp, _vp, _i, _vp, _sz, _vp, _vp, _vp]),
    "gpt2_test_quantize": (_i, [_vp, _i, _vp, _vp, _vp]),
    "gpt2_test_gemm": (_i, [_vp, _vp, _vp, _i, _i, _i, _vp]),
    "gpt2_test_gemm_bias": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp]),
    "gpt2_test_special": (_i, [_i, _u32, _sz, _vp, _vp]),
    "gpt2_test_layernorm_seq": (_i, [_vp, _i, _vp, _vp, _vp, _vp]),
    "gpt2_q8_capture_nbytes": (_sz, []),
    "gpt2_test_force_phase_kernels": (None, [_i]),
    "gpt2_test_fused_trace": (None, [_vp]),
    "gpt2_workspace_status": (_i, [_vp]),
    "gpt2_q8_capture_offsets": (_i, [_i, _i] + [ctypes.POINTER(_sz)] * 6),
    "gpt2_q8_cached_step_capture": (_i, [_vp, _vp, _sz, _u32, ctypes.c_int32, _vp, _vp, _vp, _vp]),
    "gpt2_weight_view": (_i, [_vp, _i, _i, ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                              ctypes.POINTER(_i), ctypes.POINTER(_i)]),
}

_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libgpt2mi.so; raise if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m stream_gpt_transformer_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class Gpt2Error(RuntimeError):
    def __init__(self, rc: int, what: str):
        super().__init__(f"{what} failed: {ERROR_NAMES.get(rc, rc)}")
        self.rc = rc


def _u32_array(vals: Sequence[int]):
    return (ctypes.c_uint32 * len(vals))(*[int(v) for v in vals])


# ---- direct mirrors of the C-ABI --------------------------------------------

def gpt2_packed_nbytes(flags: int) -> int:
    return int(lib().gpt2_packed_nbytes(flags))


def gpt2_workspace_nbytes() -> int:
    return int(lib().gpt2_workspace_nbytes())


def gpt2_pack_weights(ckpt_dev: int, ckpt_nbytes: int, packed_dev: int, packed_nbytes: int, flags: int,
                      stream: int = 0) -> Tuple[int, Optional[int]]:
    h = ctypes.c_void_p()
    rc = lib().gpt2_pack_weights(ckpt_dev, ckpt_nbytes, packed_dev, packed_nbytes, flags, stream, ctypes.byref(h))
    return rc, (h.value if rc == 0 else None)


def gpt2_pack_weights_grouped(ckpt_dev: int, ckpt_nbytes: int, packed_dev: int, packed_nbytes: int, flags: int,
                              q8_weight_group: int, stream: int = 0) -> Tuple[int, Optional[int]]:
    h = ctypes.c_void_p()
    rc = lib().gpt2_pack_weights_grouped(ckpt_dev, ckpt_nbytes, packed_dev, packed_nbytes, flags, q8_weight_group,
                                         stream, ctypes.byref(h))
    return rc, (h.value if rc == 0 else None)


def gpt2_q8_weight_group(model) -> int:
    return lib().gpt2_q8_weight_group(model)


def gpt2_q8_cached_step_grouped(model, input_group, cache_dev, cache_nwords, token, position, ws_dev, logits_dev,
                                stream=0) -> int:
    return lib().gpt2_q8_cached_step_grouped(model, input_group, cache_dev, cache_nwords, token & 0xFFFFFFFF,
                                             position, ws_dev, logits_dev, stream)


def gpt2_release(model: int) -> None:
    lib().gpt2_release(model)


def gpt2_cached_step(model, cache_dev, cache_nwords, token, position, ws_dev, logits_dev, stream=0) -> int:
    return lib().gpt2_cached_step(model, cache_dev, cache_nwords, token & 0xFFFFFFFF, position, ws_dev,
                                  logits_dev, stream)


def gpt2_q8_cached_step(model, cache_dev, cache_nwords, token, position, ws_dev, logits_dev, stream=0) -> int:
    return lib().gpt2_q8_cached_step(model, cache_dev, cache_nwords, token & 0xFFFFFFFF, position, ws_dev,
                                     logits_dev, stream)


def gpt2_cached_step_noalloc(model, cache_dev, cache_nwords, token, position, logits_dev, status_dev=None,
                             stream=0) -> int:
    return lib().gpt2_cached_step_noalloc(model, cache_dev, cache_nwords, token & 0xFFFFFFFF, position,
                                          logits_dev, status_dev, stream)


def gpt2_f16_cached_step(model, cache_dev, cache_nwords, token, position, ws_dev, logits_dev, stream=0) -> int:
    return lib().gpt2_f16_cached_step(model, cache_dev, cache_nwords, token & 0xFFFFFFFF, position, ws_dev,
                                      logits_dev, stream)


def gpt2_q8_cached_step_capture(model, cache_dev, cache_nwords, token, position, ws_dev, logits_dev,
                                capture_dev, stream=0) -> int:
    return lib().gpt2_q8_cached_step_capture(model, cache_dev, cache_nwords, token & 0xFFFFFFFF, position,
                                             ws_dev, logits_dev, capture_dev, stream)


def gpt2_batched_cached_step(model, caches_dev, cache_stride_words, cache_nwords: Sequence[int],
                             tokens: Sequence[int], positions: Sequence[int], ws_dev, logits_dev,
                             stream=0) -> int:
    B = len(tokens)
    nw = (ctypes.c_size_t * B)(*[int(v) for v in cache_nwords])
    tk = _u32_array([t & 0xFFFFFFFF for t in tokens])
    ps = (ctypes.c_int32 * B)(*[int(v) for v in positions])
    return lib().gpt2_batched_cached_step(model, caches_dev, cache_stride_words, ctypes.cast(nw, _vp),
                                          ctypes.cast(tk, _vp), ctypes.cast(ps, _vp), B, ws_dev, logits_dev,
                                          stream)


def gpt2_infer(model, tokens: Sequence[int], ws_dev, logits_dev, stream=0) -> int:
    tk = _u32_array([t & 0xFFFFFFFF for t in tokens]) if len(tokens) else None
    return lib().gpt2_infer(model, ctypes.cast(tk, _vp) if tk is not None else None, len(tokens), ws_dev,
                            logits_dev, stream)


def gpt2_prefill(model, tokens: Sequence[int], cache_dev, cache_capacity_nwords, ws_dev, logits_dev, stream=0) -> int:
    tk = _u32_array([t & 0xFFFFFFFF for t in tokens]) if len(tokens) else None
    return lib().gpt2_prefill(model, ctypes.cast(tk, _vp) if tk is not None else None, len(tokens), cache_dev,
                              cache_capacity_nwords, ws_dev, logits_dev, stream)


def gpt2_generate(model, cache_dev, cache_capacity_nwords, prompt: Sequence[int], n_gen, weights, ws_dev, logits_dev,
                  tokens_out_dev, status_dev, stream=0) -> int:
    tk = _u32_array([t & 0xFFFFFFFF for t in prompt]) if len(prompt) else None
    return lib().gpt2_generate(model, cache_dev, cache_capacity_nwords, ctypes.cast(tk, _vp) if tk is not None else None,
                               len(prompt), n_gen, weights, ws_dev, logits_dev, tokens_out_dev, status_dev, stream)


def gpt2_test_quantize(x_dev, n, codes_dev, scales_dev, stream=0) -> int:
    return lib().gpt2_test_quantize(x_dev, n, codes_dev, scales_dev, stream)


def gpt2_test_special(kind, first_bits, n, y_dev, stream=0) -> int:
    return lib().gpt2_test_special(kind, first_bits, n, y_dev, stream)


def gpt2_test_layernorm_seq(x_dev, rows, gamma_dev, beta_dev, y_dev, stream=0) -> int:
    return lib().gpt2_test_layernorm_seq(x_dev, rows, gamma_dev, beta_dev, y_dev, stream)


def gpt2_test_gemm(A_dev, W_dev, C_dev, M, N, K, stream=0) -> int:
    return lib().gpt2_test_gemm(A_dev, W_dev, C_dev, M, N, K, stream)


def gpt2_test_gemm_bias(A_dev, W_dev, bias_dev, C_dev, M, N, K, gelu, stream=0) -> int:
    return lib().gpt2_test_gemm_bias(A_dev, W_dev, bias_dev, C_dev, M, N, K, gelu, stream)


def gpt2_test_force_phase_kernels(on: bool) -> None:
    lib().gpt2_test_force_phase_kernels(1 if on else 0)


def gpt2_test_fused_trace(trace_dev) -> None:
    lib().gpt2_test_fused_trace(trace_dev)


def gpt2_workspace_status(ws_host_copy: bytes) -> int:
    buf = ctypes.create_string_buffer(bytes(ws_host_copy[:16]), 16)
    return lib().gpt2_workspace_status(ctypes.cast(buf, _vp))


def gpt2_q8_capture_nbytes() -> int:
    return int(lib().gpt2_q8_capture_nbytes())


def gpt2_q8_capture_offsets(layer: int, matrix: int):
    vals = [ctypes.c_size_t() for _ in range(6)]
    rc = lib().gpt2_q8_capture_offsets(layer, matrix, *[ctypes.byref(v) for v in vals])
    if rc:
        raise Gpt2Error(rc, "gpt2_q8_capture_offsets")
    return dict(zip(("base", "in", "codes", "scales", "acc", "out"), (v.value for v in vals)))


def gpt2_weight_view(model, layer: int, matrix: int):
    f, c, s = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
    r, k = ctypes.c_int(), ctypes.c_int()
    rc = lib().gpt2_weight_view(model, layer, matrix, ctypes.byref(f), ctypes.byref(c), ctypes.byref(s),
                                ctypes.byref(r), ctypes.byref(k))
    if rc:
        raise Gpt2Error(rc, "gpt2_weight_view")
    return dict(f32=f.value, codes=c.value, scales=s.value, rows=r.value, cols=k.value)


# ---- convenience: torch-owned device memory ---------------------------------

def _stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


class Model:
    """A packed model whose device memory (packed weights, workspace) torch owns."""

    def __init__(self, ckpt_dev, flags: int = GPT2_PACK_F32, q8_weight_group: int = 64):
        """q8_weight_group: the int8 weight-scale group (gpt2_pack_weights_grouped)."""
        import torch
        self.flags = flags
        n = gpt2_packed_nbytes(flags)
        self.packed = torch.empty(n, dtype=torch.uint8, device=ckpt_dev.device)
        self.ws = torch.zeros(gpt2_workspace_nbytes(), dtype=torch.uint8, device=ckpt_dev.device)
        rc, h = gpt2_pack_weights_grouped(ckpt_dev.data_ptr(), ckpt_dev.numel() * ckpt_dev.element_size(),
                                          self.packed.data_ptr(), n, flags, q8_weight_group, _stream())
        if rc:
            raise Gpt2Error(rc, "gpt2_pack_weights_grouped")
        self.handle = h

    def close(self) -> None:
        if getattr(self, "handle", None):
            gpt2_release(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def status(self) -> int:
        """Error word of this model's workspace (0 = fine)."""
        return gpt2_workspace_status(self.ws[:16].cpu().numpy().tobytes())

    def new_cache(self, positions: int = GPT2_MAX_POS, batch: int = 0):
        import torch
        shape = (positions * GPT2_CACHE_WORDS_PER_POS,) if batch == 0 else (batch, positions * GPT2_CACHE_WORDS_PER_POS)
        return torch.zeros(shape, dtype=torch.float32, device=self.packed.device)

    def step(self, cache, pos: int, token: int, logits, q8: bool = False, f16: bool = False,
             input_group: int = 64) -> None:
        """One cached step (int8 with q8; input_group: its input-scale group)."""
        if q8 and input_group != 64:
            rc = gpt2_q8_cached_step_grouped(self.handle, input_group, cache.data_ptr(),
                                             pos * GPT2_CACHE_WORDS_PER_POS, token, pos, self.ws.data_ptr(),
                                             logits.data_ptr(), _stream())
            if rc:
                raise Gpt2Error(rc, "gpt2_q8_cached_step_grouped")
            return
        fn = gpt2_q8_cached_step if q8 else gpt2_f16_cached_step if f16 else gpt2_cached_step
        rc = fn(self.handle, cache.data_ptr(), pos * GPT2_CACHE_WORDS_PER_POS, token, pos, self.ws.data_ptr(),
                logits.data_ptr(), _stream())
        if rc:
            raise Gpt2Error(rc, fn.__name__)

    def batched_step(self, caches, positions, tokens, logits) -> None:
        B = len(tokens)
        rc = gpt2_batched_cached_step(self.handle, caches.data_ptr(), caches.shape[1],
                                      [p * GPT2_CACHE_WORDS_PER_POS for p in positions], tokens, positions,
                                      self.ws.data_ptr(), logits.data_ptr(), _stream())
        if rc:
            raise Gpt2Error(rc, "gpt2_batched_cached_step")

    def generate(self, cache, prompt, n_gen: int, logits, tokens_out, status, q8: bool = False,
                 f16: bool = False) -> None:
        """Greedy generation on the device (gpt2_generate): cache, logits, tokens_out
        (uint32 or int32, n_gen) and status (int32, 1) are device tensors."""
        weights = GPT2_WEIGHTS_Q8 if q8 else GPT2_WEIGHTS_F16 if f16 else GPT2_WEIGHTS_F32
        rc = gpt2_generate(self.handle, cache.data_ptr(), cache.numel(), list(prompt), n_gen, weights,
                           self.ws.data_ptr(), logits.data_ptr(), tokens_out.data_ptr(), status.data_ptr(), _stream())
        if rc:
            raise Gpt2Error(rc, "gpt2_generate")

    def prefill(self, tokens, cache, logits) -> None:
        """gpt2_prefill: infer over tokens, also filling cache (device float32) for them."""
        rc = gpt2_prefill(self.handle, list(tokens), cache.data_ptr(), cache.numel(), self.ws.data_ptr(),
                          logits.data_ptr(), _stream())
        if rc:
            raise Gpt2Error(rc, "gpt2_prefill")

    def infer(self, tokens, logits) -> None:
        rc = gpt2_infer(self.handle, list(tokens), self.ws.data_ptr(), logits.data_ptr(), _stream())
        if rc:
            raise Gpt2Error(rc, "gpt2_infer")
