// Device-side building blocks of the decode step.
//
// Every output value of the decode path is defined by one of the functions here,
// with a fixed data-to-lane mapping and a fixed reduction tree, independent of
// the grid that calls it.  The batch-1 step, the fused batch-1 step and the
// batched step all call these functions, so a session gives the same bits in
// any of them (batch invariance, the muInference page's batch-invariance
// paragraph; gpt2.s page: the same addition order gives identical output for any
// process count).  The library is built with -ffp-contract=off; every fused
// multiply-add below is written out as fmaf.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "layout.hpp"

namespace g2 {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef int i4 __attribute__((ext_vector_type(4)));

// All 64 lanes end with the same value: at each butterfly step lanes l and l^m add
// the same two operands (in swapped order; addition commutes exactly).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = v + __shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// ---- lane fragments ---------------------------------------------------------
// A K-vector (K = 256*NI) is spread over one wavefront as NI float4 per lane:
// lane l holds elements 256*i + 4*l + e (i < NI, e < 4).  A weight row uses the
// same mapping, so a row is read with NI fully coalesced 1 KB wave loads.
template <int NI>
__device__ __forceinline__ void load_frag(f4 (&x)[NI], const float* __restrict__ src) {
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < NI; ++i) x[i] = *(const f4*)(src + 256 * i + 4 * l);
}
template <int NI>
__device__ __forceinline__ void store_frag(float* __restrict__ dst, const f4 (&x)[NI]) {
  const int l = lane_id();
#pragma unroll
  for (int i = 0; i < NI; ++i) *(f4*)(dst + 256 * i + 4 * l) = x[i];
}

// LayerNorm of a 768-vector held as a fragment (one wave):
// mean = (sum x)/768, d = x - mean, var = (sum d*d)/768, r = 1/sqrt(var + 1e-5),
// y = (d*r)*gamma + beta.  Each lane sums its 12 values in (i, e) order, then the
// butterfly combines lanes.
__device__ __forceinline__ void layernorm_frag(f4 (&x)[3], const float* __restrict__ gamma,
                                               const float* __restrict__ beta) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 3; ++i) { s = s + x[i].x; s = s + x[i].y; s = s + x[i].z; s = s + x[i].w; }
  s = wave_sum(s);
  const float mean = s / 768.0f;
  float v = 0.0f;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    x[i] = x[i] - mean;
    v = v + x[i].x * x[i].x; v = v + x[i].y * x[i].y; v = v + x[i].z * x[i].z; v = v + x[i].w * x[i].w;
  }
  v = wave_sum(v);
  const float var = v / 768.0f;
  const float r = 1.0f / sqrtf(var + 1e-5f);
  f4 g[3], b[3];
  load_frag<3>(g, gamma);
  load_frag<3>(b, beta);
#pragma unroll
  for (int i = 0; i < 3; ++i) x[i] = (x[i] * r) * g[i] + b[i];
}

// One output of an fp32 projection: lane l accumulates its 4*NI products with an
// explicit fmaf chain in (i, e) order, then the butterfly sums the 64 lane partials.
// The returned value (identical in every lane) excludes the bias.
template <int NI>
__device__ __forceinline__ float dot_frag(const f4 (&w)[NI], const f4 (&x)[NI]) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    acc = fmaf(w[i].x, x[i].x, acc);
    acc = fmaf(w[i].y, x[i].y, acc);
    acc = fmaf(w[i].z, x[i].z, acc);
    acc = fmaf(w[i].w, x[i].w, acc);
  }
  return wave_sum(acc);
}

// tanh form of GELU: 0.5*u*(1 + tanh(sqrt(2/pi)*(u + 0.044715*u^3))).
__device__ __forceinline__ float gelu_tanh(float u) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi) rounded to binary32
  const float inner = u + 0.044715f * (u * u * u);
  const float t = tanhf(c * inner);
  return (0.5f * u) * (1.0f + t);
}

// ---- attention (one session, one head) --------------------------------------
// 128 threads (two wavefronts); thread t owns key t.  With npos keys (1..128):
//   s_t = fmaf-chain over d of q_d*K_t,d, times 0.125 (1/sqrt(64));
//   m = max_t s_t;  e_t = exp(s_t - m) (0 for t >= npos);
//   Z = wave-butterfly sum of each wave's e, then Z = Z_wave0 + Z_wave1;
//   w_t = e_t / Z;
//   a_d = (fmaf-chain over t < 64 of w_t*V_t,d) + (fmaf-chain over 64 <= t < npos).
struct AttnSmem {
  float k[PMAX][DH + 1];  // padded row: lanes reading K_t,d for consecutive t avoid bank clashes
  float v[PMAX][DH];
  float q[DH];
  float w[PMAX];
  float red[4];
  float part[DH];
};

// Stage npos key/value rows of one head into LDS.  Row t of the keys is at
// kv(t) (64 keys), its values at kv(t) + D.  Called by all 128 threads.
template <class RowPtr>
__device__ __forceinline__ void attn_stage(AttnSmem& sm, RowPtr kv, int npos, const float* q) {
  const int t = threadIdx.x;
  for (int idx = t; idx < npos * 16; idx += 128) {
    const int j = idx >> 4, c = (idx & 15) * 4;
    const float* row = kv(j);
    const f4 kk = *(const f4*)(row + c);
    const f4 vv = *(const f4*)(row + D + c);
    sm.k[j][c + 0] = kk.x; sm.k[j][c + 1] = kk.y; sm.k[j][c + 2] = kk.z; sm.k[j][c + 3] = kk.w;
    *(f4*)&sm.v[j][c] = vv;
  }
  if (t < DH) sm.q[t] = q[t];
}

// Returns a_d in threads 0..63 (d = thread index); other threads return 0.
__device__ __forceinline__ float attn_compute(AttnSmem& sm, int npos) {
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  float s = -INFINITY;
  if (t < npos) {
    float acc = 0.0f;
#pragma unroll 16
    for (int d = 0; d < DH; ++d) acc = fmaf(sm.q[d], sm.k[t][d], acc);
    s = acc * 0.125f;
  }
  const float mw = wave_max(s);
  if (lane == 0) sm.red[wv] = mw;
  __syncthreads();
  const float m = fmaxf(sm.red[0], sm.red[1]);
  const float e = t < npos ? expf(s - m) : 0.0f;
  const float zw = wave_sum(e);
  if (lane == 0) sm.red[2 + wv] = zw;
  __syncthreads();
  const float Z = sm.red[2] + sm.red[3];
  sm.w[t] = e / Z;
  __syncthreads();
  float acc = 0.0f;
  const int j1 = min(npos, 64 * wv + 64);
  for (int j = 64 * wv; j < j1; ++j) acc = fmaf(sm.w[j], sm.v[j][lane], acc);
  if (wv == 1) sm.part[lane] = acc;
  __syncthreads();
  return wv == 0 ? acc + sm.part[lane] : 0.0f;
}

// ---- int8 group-64 quantizer (marXiv 2609.00018 abstract) --------------------
// One group of 64 values, one per lane: m = max|x| (exact), s = m/127 (correctly
// rounded), code = clamp(rint(x/s), -127, 127) with rint rounding half to even;
// m == 0 gives s = 0 and code 0; a NaN code is 0.
__device__ __forceinline__ int quant_lane(float x, float& s_out) {
  const float m = wave_max(fabsf(x));
  if (m == 0.0f) { s_out = 0.0f; return 0; }
  const float s = m / 127.0f;
  s_out = s;
  float q = rintf(x / s);
  if (q != q) q = 0.0f;
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return (int)q;
}

}  // namespace g2
