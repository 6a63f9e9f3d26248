// Internal interface between the C-ABI layer and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "layout.hpp"

namespace g2 {

// Device pointers into a packed weight buffer.
struct Weights {
  const float* wte;    // [V][D] token embeddings = tied head matrix
  const float* wpe;    // [PMAX][D]
  const float* small;  // per-layer LayerNorm parameters and biases (sp:: offsets)
  const float* f32;    // per-layer [out][in] fp32 matrices, or null
  const int8_t* q8c;   // per-layer [out][in] int8 codes, then the head [V][D], or null
  const float* q8s;    // per-layer [out][in/64] scales, then the head [V][D/64], or null
  const uint16_t* f16; // per-layer [out][in] binary16 matrices, then the token table [V][D], or null
};

__host__ __device__ inline const float* f32_mat(const Weights& w, int layer, int m) {
  return w.f32 + (size_t)layer * LAYER_ELEMS + mat_elem_off(m);
}
__host__ __device__ inline const int8_t* q8_codes(const Weights& w, int layer, int m) {
  return m == M_HEAD ? w.q8c + (size_t)L * LAYER_ELEMS : w.q8c + (size_t)layer * LAYER_ELEMS + mat_elem_off(m);
}
__host__ __device__ inline const float* q8_scales(const Weights& w, int layer, int m) {
  return m == M_HEAD ? w.q8s + (size_t)L * LAYER_SCALES : w.q8s + (size_t)layer * LAYER_SCALES + mat_scale_off(m);
}
__host__ __device__ inline const uint16_t* f16_mat(const Weights& w, int layer, int m) {
  return m == M_HEAD ? w.f16 + (size_t)L * LAYER_ELEMS : w.f16 + (size_t)layer * LAYER_ELEMS + mat_elem_off(m);
}
__host__ __device__ inline const float* small_p(const Weights& w, int layer, int off) {
  return w.small + (size_t)layer * sp::PER_LAYER + off;
}

// Sessions advanced by one decode launch (kernel argument, <= 4 KB).
struct Sessions {
  int B;
  uint32_t tok[MAX_BATCH];
  int32_t pos[MAX_BATCH];
};

// Workspace pointers.
struct Work {
  uint32_t* header;
  float* x;    // [B][D] residual stream
  float* qkv;  // [B][3D]
  float* att;  // [B][D]
  float* g;    // [B][F]
  unsigned long long* ll;
  float *pf_x, *pf_h, *pf_qkv, *pf_att, *pf_u, *pf_part;
  // A workspace that every call shares (the library's own scratch): the single-launch
  // step reports its error word into step_status (device, may be null) and clears it.
  bool self_clearing;
  int32_t* step_status;
};

Work work_ptrs(void* ws, int max_batch);

hipError_t launch_pack(const float* ckpt, char* packed, int flags, hipStream_t s, int q8_group = 64);
// Header word of the workspace that carries the token a generation step is fed
// (written by k_argmax, read by the step's embedding).
constexpr int HDR_WORD_NEXT_TOKEN = 3;

// Stored weight format of a step: fp32, int8 group-64, or binary16 (computed in fp32).
enum WFmt { WF_F32 = 0, WF_Q8 = 1, WF_F16 = 2 };

// tokp: when given, session 0's token is read from device memory at run time
// instead of ss.tok[0] / token.  h16: the binary16 weights (batch 1 only).
hipError_t launch_step_f32(const Weights& w, const Work& k, const Sessions& ss, float* caches,
                           size_t cache_stride, float* logits, hipStream_t s, const uint32_t* tokp = nullptr,
                           bool h16 = false);
// qx, qw: the input- and weight-scale groups in units of 64 coordinates (64*q
// dividing 768, or 0 for the whole row); the weights must have been packed with qw.
hipError_t launch_step_q8(const Weights& w, const Work& k, const Sessions& ss, float* cache,
                          float* logits, char* capture, hipStream_t s, const uint32_t* tokp = nullptr, int qx = 1,
                          int qw = 1);
hipError_t launch_argmax(const float* logits, uint32_t* next, uint32_t* tokens_out, int32_t* status, int step,
                         hipStream_t s);
// cache (or null): the key/value rows of positions 0..n-1 are also written there
// in the cachedStep layout.
hipError_t launch_infer(const Weights& w, const Work& k, const uint32_t* toks, int n, float* logits,
                        hipStream_t s, float* cache = nullptr);
// device_token: a generation step, whose token is the workspace header's word
// HDR_WORD_NEXT_TOKEN (a separate kernel instantiation; capture must be null).
hipError_t launch_fused(WFmt f, const Weights& w, const Work& k, uint32_t token, int32_t pos, float* cache,
                        float* logits, char* capture, hipStream_t s, bool* used, bool device_token = false);
extern bool g_force_phase_kernels;
extern uint64_t* g_fused_trace;
hipError_t launch_special_bits(int kind, uint32_t first, long long n, float* y, hipStream_t s);
hipError_t launch_layernorm_seq(const float* x, int rows, const float* gamma, const float* beta, float* y,
                                hipStream_t s);
hipError_t launch_quantize(const float* x, int n, int8_t* codes, float* scales, hipStream_t s);
hipError_t launch_gemm16_test(const float* A, const float* W, const float* bias, float* C, int M, int N, int K,
                              bool gelu, hipStream_t s);
hipError_t launch_gemm_test(const float* A, const float* W, float* C, int M, int N, int K, hipStream_t s);

}  // namespace g2
