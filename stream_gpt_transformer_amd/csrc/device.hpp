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
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

// Four binary16 weights widened to binary32 (exact: every binary16 value is a
// binary32 value).
__device__ __forceinline__ f4 widen(const h4 h) { return __builtin_convertvector(h, f4); }

// ---- cross-lane reductions on DPP ---------------------------------------------
// Lane moves inside one VALU instruction (GFX9 data-parallel primitives), with no
// trip through the LDS crossbar.  quad_perm [1,0,3,2] and [2,3,0,1] swap lanes at
// distance 1 and 2; row_half_mirror and row_mirror reverse 8- and 16-lane groups,
// which acts as a swap at distance 4 and 8 once the quads (then the 8-lane halves)
// hold equal values; row_bcast:15 adds row r-1's last lane into row r (rows 1, 3),
// row_bcast:31 adds lane 31 into rows 2 and 3 (the prefix scans use these two).
// Across rows the reductions use gfx950's row and half-wave swaps instead.
enum : int {
  DPP_QUAD_1032 = 0xB1,
  DPP_QUAD_2301 = 0x4E,
  DPP_ROW_SL4 = 0x104,   // row_shl:4 (lane l of a row reads lane l + 4)
  DPP_ROW_SL8 = 0x108,
  DPP_ROW_SL12 = 0x10C,
  DPP_QUAD_3210 = 0x1B,
  DPP_ROW_MIRROR = 0x140,
  DPP_ROW_HALF_MIRROR = 0x141,
  DPP_ROW_BCAST15 = 0x142,
  DPP_ROW_BCAST31 = 0x143,
};
// With every row enabled (the quad permutes and mirrors, whose source lanes all
// exist) the move has no old value, so the compiler folds it into the VALU op that
// consumes it (one v_add_f32_dpp instead of a move and an add).  With a partial row
// mask the rows left out keep their own value.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_f(float v) {
  const int i = __float_as_int(v);
  if constexpr (ROWS == 0xf) return __int_as_float(__builtin_amdgcn_mov_dpp(i, CTRL, 0xf, 0xf, true));
  else return __int_as_float(__builtin_amdgcn_update_dpp(i, i, CTRL, ROWS, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, true);
}
__device__ __forceinline__ float bcast_lane(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over each 16-lane row; every lane of the row ends with the row's value
// (the two operands of each step are equal in every lane of a pair, in swapped
// order, and addition commutes exactly).
__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp_f<DPP_QUAD_1032>(v);
  v = v + dpp_f<DPP_QUAD_2301>(v);
  v = v + dpp_f<DPP_ROW_HALF_MIRROR>(v);
  v = v + dpp_f<DPP_ROW_MIRROR>(v);
  return v;
}
// Rows 0 and 1 (and 2 and 3) exchanged, then the two 32-lane halves (gfx950
// v_permlane16_swap / v_permlane32_swap on two copies of v): a + b holds, in every
// lane, the combination of the lane's row (half) with its partner row (half).
__device__ __forceinline__ float swap_rows_add(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_halves_add(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_rows_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Sum of the 64 lanes: row sums r0..r3 as above, then (r0 + r1) + (r2 + r3) (each
// add's operands in either order: the same value), in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  return swap_halves_add(swap_rows_add(row16_sum(v)));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_1032>(v));
  v = fmaxf(v, dpp_f<DPP_QUAD_2301>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v));
  v = fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v));
  return swap_halves_max(swap_rows_max(v));
}
// N independent wave sums in lock step (the same tree as wave_sum for each value,
// interleaved so that the lane moves of one hide the latency of the others).
template <int N>
__device__ __forceinline__ void wave_sum_n(float (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = v[k] + dpp_f<DPP_QUAD_1032>(v[k]);
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = v[k] + dpp_f<DPP_QUAD_2301>(v[k]);
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = v[k] + dpp_f<DPP_ROW_HALF_MIRROR>(v[k]);
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = v[k] + dpp_f<DPP_ROW_MIRROR>(v[k]);
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = swap_rows_add(v[k]);
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = swap_halves_add(v[k]);
}
// The 16-lane tree of row16_sum evaluated inside one lane on s[0..15] (s[j] being
// what lane j of the row holds): the same value, by commutativity of each add.
__device__ __forceinline__ float row16_tree(const float (&s)[16]) {
  const float a = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
  const float b = ((s[8] + s[9]) + (s[10] + s[11])) + ((s[12] + s[13]) + (s[14] + s[15]));
  return a + b;
}
// The lane part of dot_q16: the fmaf chain over one float4.
__device__ __forceinline__ float fma4(const f4 w, const f4 x) {
  float acc = 0.0f;
  acc = fmaf(w.x, x.x, acc);
  acc = fmaf(w.y, x.y, acc);
  acc = fmaf(w.z, x.z, acc);
  acc = fmaf(w.w, x.w, acc);
  return acc;
}

// Exact integer sum over each 4-lane quad (every lane of the quad gets it).
__device__ __forceinline__ int quad_sum(int p) {
  p += dpp_i<DPP_QUAD_1032>(p);
  p += dpp_i<DPP_QUAD_2301>(p);
  return p;
}
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }
// The lane index through an empty asm: address arithmetic derived from it is redone
// where it is used, instead of being hoisted out of a loop and kept live in
// registers (the weight-load helpers call it).
__device__ __forceinline__ int lane_id_fresh() {
  int l = (int)(threadIdx.x & 63);
  asm volatile("" : "+v"(l));
  return l;
}

// ---- many outputs at once ----------------------------------------------------
// row16_sum's tree for N outputs (a power of two, <= 16) together, transposed over
// the 16 lanes of each row.  Level k pairs lane b with lane b ^ m_k (m = 1, 3, 7,
// 15: quad_perm [1,0,3,2], quad_perm [3,2,1,0], row_half_mirror, row_mirror), which
// lies in the other 2^k-lane block of the same 2^(k+1)-lane block, as row16_sum's
// level k does.  While outputs remain to split, the two partners hold partial sums
// of the same outputs (over their two blocks); each keeps the half of them whose
// output-index bit k equals c_k(lane) and adds its partner's copy of that half, the
// partner keeping the other half (c_0 = b0^b1, c_1 = b1^b2, c_2 = b2^b3, c_3 = b3 for
// the row's lane bits b: partners differ in c_k and agree in the earlier ones).
// After the split levels the partners hold the same output and add as row16_sum.
// Every add joins the same two block sums as in row16_sum, so each result is bit
// for bit row16_sum's value of that output; lane t of every row ends with output
// treduce_out<N>(t), the sum over its own row.
__device__ __forceinline__ int treduce_c(int t, int k) { return k < 3 ? ((t >> k) ^ (t >> (k + 1))) & 1 : (t >> 3) & 1; }
template <int N>
__device__ __forceinline__ int treduce_out(int t) {
  int o = 0;
#pragma unroll
  for (int k = 0; (1 << k) < N; ++k) o |= treduce_c(t, k) << k;
  return o;
}
// The first lane t of a row with treduce_out<N>(t) == o (a compile-time constant).
template <int N>
__host__ __device__ constexpr int treduce_lane(int o) {
  for (int t = 0; t < 16; ++t) {
    int oo = 0;
    for (int k = 0; (1 << k) < N; ++k) oo |= (k < 3 ? ((t >> k) ^ (t >> (k + 1))) & 1 : (t >> 3) & 1) << k;
    if (oo == o) return t;
  }
  return -1;
}
template <int CTRL, int N>
__device__ __forceinline__ void treduce_level(float (&a)[16], int& n, bool c) {
  if (n >= 2) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      if (2 * i < n) {
        const float x = c ? a[2 * i + 1] : a[2 * i];
        const float y = c ? a[2 * i] : a[2 * i + 1];
        a[i] = x + dpp_f<CTRL>(y);
      }
    }
    n /= 2;
  } else {
    a[0] = a[0] + dpp_f<CTRL>(a[0]);
  }
}
template <int N>
__device__ __forceinline__ float row_treduce(const float (&v)[N]) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "outputs per row reduction");
  const int t = lane_id() & 15;
  float a[16];
#pragma unroll
  for (int j = 0; j < N; ++j) a[j] = v[j];
  int n = N;
  treduce_level<DPP_QUAD_1032, N>(a, n, treduce_c(t, 0));
  treduce_level<DPP_QUAD_3210, N>(a, n, treduce_c(t, 1));
  treduce_level<DPP_ROW_HALF_MIRROR, N>(a, n, treduce_c(t, 2));
  treduce_level<DPP_ROW_MIRROR, N>(a, n, treduce_c(t, 3));
  return a[0];
}
// wave_sum's tree for N outputs together: lane t of every row holds the 64-lane sum
// of output treduce_out<N>(t).
template <int N>
__device__ __forceinline__ float wave_treduce(const float (&v)[N]) {
  return swap_halves_add(swap_rows_add(row_treduce<N>(v)));
}
// Row r's value of v in the lanes of row 0 (r = 1, 2, 3; other rows: any value).
__device__ __forceinline__ float row1_to_row0(float v) {
  return __uint_as_float(__builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false)[1]);
}
__device__ __forceinline__ float row2_to_row0(float v) {
  return __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false)[1]);
}
__device__ __forceinline__ float row3_to_row0(float v) { return row2_to_row0(row1_to_row0(v)); }

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
// y = fmaf(d*r, gamma, beta).  Each lane sums its 12 values as a tree (pairs inside
// each float4, then the float4 sums), the squares as an fmaf chain per float4, then
// the wave_sum combines lanes; the statistics are products by 1/768 and the hardware
// reciprocal square root (within an ulp or two of s/768 and 1/sqrt).  Every fp32 path
// uses this same function, so they stay identical to each other.
__device__ __forceinline__ void layernorm_frag(f4 (&x)[3], const float* __restrict__ gamma,
                                               const float* __restrict__ beta) {
  // gamma and beta first, so their reads overlap the statistics
  f4 g[3], b[3];
  load_frag<3>(g, gamma);
  load_frag<3>(b, beta);
  float s = ((x[0].x + x[0].y) + (x[0].z + x[0].w)) + ((x[1].x + x[1].y) + (x[1].z + x[1].w));
  s = s + ((x[2].x + x[2].y) + (x[2].z + x[2].w));
  s = wave_sum(s);
  const float mean = s * (1.0f / 768.0f);
#pragma unroll
  for (int i = 0; i < 3; ++i) x[i] = x[i] - mean;
  float q[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) q[i] = fmaf(x[i].w, x[i].w, fmaf(x[i].z, x[i].z, fmaf(x[i].y, x[i].y, x[i].x * x[i].x)));
  float v = (q[0] + q[1]) + q[2];
  v = wave_sum(v);
  const float var = v * (1.0f / 768.0f);
  const float r = __builtin_amdgcn_rsqf(var + 1e-5f);
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    x[i].x = fmaf(x[i].x * r, g[i].x, b[i].x);
    x[i].y = fmaf(x[i].y * r, g[i].y, b[i].y);
    x[i].z = fmaf(x[i].z * r, g[i].z, b[i].z);
    x[i].w = fmaf(x[i].w * r, g[i].w, b[i].w);
  }
}

// One output of an fp32 projection: lane l accumulates its 4*NI products with an
// explicit fmaf chain in (i, e) order, then wave_sum adds the 64 lane partials.
// The returned value (identical in every lane) excludes the bias.
// dot_frag's lane part (before wave_sum).
template <int NI>
__device__ __forceinline__ float dot_lane(const f4* w, const f4 (&x)[NI]) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    acc = fmaf(w[i].x, x[i].x, acc);
    acc = fmaf(w[i].y, x[i].y, acc);
    acc = fmaf(w[i].z, x[i].z, acc);
    acc = fmaf(w[i].w, x[i].w, acc);
  }
  return acc;
}
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

// One 64-input group dot on a quarter wave: lane j of the quarter holds inputs
// 4j..4j+3 of the group, runs an fmaf chain over them, and row16_sum over the 16
// lanes of the quarter sums the partials (all 16 lanes end with the value).
__device__ __forceinline__ float dot_q16(const f4 w, const f4 x) {
  float acc = 0.0f;
  acc = fmaf(w.x, x.x, acc);
  acc = fmaf(w.y, x.y, acc);
  acc = fmaf(w.z, x.z, acc);
  acc = fmaf(w.w, x.w, acc);
  return row16_sum(acc);
}
__device__ __forceinline__ float lane_val(float v, int lane) { return bcast_lane(v, lane); }

// The fp32 output projection as a sum over heads.  In the lane-fragment layout the
// 64 inputs of head h = 4i + q sit in quarter q of fragment i, so p_h = dot_q16 of
// that quarter; then y = 0, y = y + p_h for h = 0..11 (bias excluded).
__device__ __forceinline__ float o_row(const f4 (&w)[3], const f4 (&x)[3]) {
  float p[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) p[i] = dot_q16(w[i], x[i]);
  float y = 0.0f;
#pragma unroll
  for (int h = 0; h < H; ++h) y = y + lane_val(p[h / 4], 16 * (h % 4));
  return y;
}

// The fp32 MLP projection (3072 inputs) as a sum over eight slices of 384 inputs
// (six 64-input groups each): q_g = dot_q16 of group g (quarter g%4 of fragment
// g/4); p_s = q_6s + q_6s+1 + ... + q_6s+5 in order; y = 0, y = y + p_s for
// s = 0..7 (bias excluded).
constexpr int PR_SLICES = 8;
constexpr int PR_SLICE_GROUPS = F / 64 / PR_SLICES;  // 6
__device__ __forceinline__ float pr_row(const f4 (&w)[12], const f4 (&x)[12]) {
  float q[12];
#pragma unroll
  for (int f = 0; f < 12; ++f) q[f] = dot_q16(w[f], x[f]);
  float y = 0.0f;
#pragma unroll
  for (int s = 0; s < PR_SLICES; ++s) {
    const int g0 = PR_SLICE_GROUPS * s;
    float p = lane_val(q[g0 / 4], 16 * (g0 % 4));
#pragma unroll
    for (int k = 1; k < PR_SLICE_GROUPS; ++k) p = p + lane_val(q[(g0 + k) / 4], 16 * ((g0 + k) % 4));
    y = y + p;
  }
  return y;
}

// Ordered binary32 exponential (LeanExe GPT-2 README, numerical functions: an
// ordered binary32 exponential approximation; muInference page, IEEE-ops table:
// range reduction, Taylor polynomial, 2^k as a bit pattern, only correctly rounded
// operations).  Each line is one rounded binary32 operation, in this order:
// k = rint(x*log2 e); r = (x - k*ln2_hi) - k*ln2_lo with ln2_hi = 0x3f317200 (k*ln2_hi
// exact); degree-7 Taylor polynomial of e^r by Horner from 1/5040 down to 1; times
// 2^k from its bit pattern.  NaN passes through, x >= 88.72283935546875 gives +inf,
// x < -87 gives 0 (so no result is subnormal).
__device__ __forceinline__ float exp_spec(float x) {
  if (x != x) return x;
  if (x >= 88.72283935546875f) return INFINITY;
  if (x < -87.0f) return 0.0f;
  const float k = rintf(x * 1.44269502162933349609375f);
  const float r = (x - k * 0.693145751953125f) - k * 1.428606765330187e-06f;
  float p = 1.0f / 5040.0f;
  p = p * r + 1.0f / 720.0f;
  p = p * r + 1.0f / 120.0f;
  p = p * r + 1.0f / 24.0f;
  p = p * r + 1.0f / 6.0f;
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  int ki = (int)k;
  if (ki == 128) {
    p = p * 2.0f;
    ki = 127;
  }
  return p * __uint_as_float((unsigned)(ki + 127) << 23);
}

// tanh(z) = 1 - 2/(exp(2|z|) + 1), with the sign of z.
__device__ __forceinline__ float tanh_spec(float z) {
  const float e = exp_spec(2.0f * fabsf(z));
  const float t = 1.0f - 2.0f / (e + 1.0f);
  return z < 0.0f ? -t : t;
}

// dot_frag with the input fragment read from LDS one float4 at a time (same fmaf
// chain and wave_sum, so the same value; fewer live registers).
template <int NI>
__device__ __forceinline__ float dot_lds(const f4 (&w)[NI], const float* xs) {
  const int l = lane_id();
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const f4 x = *(const f4*)(xs + 256 * i + 4 * l);
    acc = fmaf(w[i].x, x.x, acc);
    acc = fmaf(w[i].y, x.y, acc);
    acc = fmaf(w[i].z, x.z, acc);
    acc = fmaf(w[i].w, x.w, acc);
  }
  return wave_sum(acc);
}

// tanh form of GELU: 0.5*u*(1 + tanh(sqrt(2/pi)*(u + 0.044715*u^3))).
__device__ __forceinline__ float gelu_tanh(float u) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi) rounded to binary32
  const float inner = u + 0.044715f * (u * u * u);
  const float t = tanh_spec(c * inner);
  return (0.5f * u) * (1.0f + t);
}

// The binary32 path's exponential for arguments <= 0 (softmax): the hardware base-2
// exponential of x*log2(e), within a few ulp of exp_spec.
__device__ __forceinline__ float exp_f32(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// The binary32 path's GELU: the same tanh form, with exp(2|z|) from the hardware
// base-2 exponential and 2/(e + 1) from the hardware reciprocal (a few ulp from
// gelu_tanh).  The int8 path keeps gelu_tanh, whose exponential is the specified one;
// every binary32 path uses this one, so they stay identical to each other.
__device__ __forceinline__ float gelu_f32(float u) {
  const float c = 0.7978845608028654f;
  const float inner = u + 0.044715f * (u * u * u);
  const float z = c * inner;
  const float e = __builtin_amdgcn_exp2f(2.8853900817779268f * fabsf(z));  // 2 log2(e) |z|
  const float t0 = 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
  const float t = z < 0.0f ? -t0 : t0;
  return (0.5f * u) * (1.0f + t);
}

// ---- sequential-order LayerNorm (the int8 path) -----------------------------
// The int8 path quantizes LayerNorm outputs, so a one-ulp difference in an output
// can move a code across a rounding boundary; its LayerNorm therefore takes every
// sum sequentially in index order, one rounding per operation, as the oracle does:
//   mean = (((0 + x_0) + x_1) + ... + x_767) / 768;  d_i = x_i - mean;
//   var = (((0 + d_0*d_0) + d_1*d_1) + ...) / 768;  r = 1/sqrt(var + 1e-5);
//   y_i = (d_i*r)*gamma_i + beta_i.
// A chain of dependent adds is the cost: a wave reads the next 32 values from LDS
// (broadcast reads) while it adds the current 32, so the chain never waits for LDS.
__device__ __forceinline__ void lds_load32(f4 (&v)[8], const float* p) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = *(const f4*)(p + 4 * i);
}
__device__ __forceinline__ void seq_add32(float& s, const f4 (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s = s + v[i].x;
    s = s + v[i].y;
    s = s + v[i].z;
    s = s + v[i].w;
  }
}
// ---- the same sequential sums, evaluated by a whole workgroup -----------------
// seq_sum768_wg returns (((0 + t_0) + t_1) + ... + t_767), one binary32 rounding per
// add, bit for bit the sequential loop's value for finite t, in about half the
// latency of one wave running the loop.  All 512 threads (8 waves) of the
// workgroup call it.
//  1. Estimates: every wave forms the binary64 prefix sums of t (lane i sums
//     t[12i..12i+11], then an inclusive scan over the lanes) and rounds the prefix
//     at each segment start to binary32: E_k for segment k = t[96k..96k+95], k < 8.
//  2. Candidates: lane j of wave k runs the ordered chain of segment k from the
//     binary32 value j - 32 steps away from E_k (steps through consecutive
//     representable values) and stores where it ends.
//  3. Walk: with S_0 = +0 the true start of segment 0, wave 0 follows the segments
//     in order.  If S_k is one of the 64 candidates of segment k, the chain that
//     started exactly at S_k ended at S_(k+1); otherwise the wave runs the chain
//     of segment k from S_k itself.
// Every chain is the loop's own sequence of roundings from its start value, and a
// candidate is used only when its start equals the loop's running sum, so the
// estimates affect only how often step 3 runs a chain itself.  (The running sum
// is never -0: it starts at +0 and a round-to-nearest sum is -0 only when both
// operands are.)  tab is SEQ_TAB_FLOATS floats of LDS scratch; t must be in LDS
// and not change during the call; the call has two workgroup barriers, and tab
// may be written again after the caller's next one.
__device__ __forceinline__ int f_ord(int bits) { return bits < 0 ? -(bits & 0x7fffffff) : bits; }
__device__ __forceinline__ int f_from_ord(int o) { return o < 0 ? (int)(0x80000000u | (uint32_t)(-o)) : o; }
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_d0(double v) {  // lanes without a source read 0
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, ROWS, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (uint32_t)lo);
}
// s + t[0] + ... + t[95] in order (t in LDS; 32 values in flight while 32 are added).
__device__ __forceinline__ float seq_chain96(float s, const float* t) {
  f4 a[8], b[8];
  lds_load32(a, t);
  lds_load32(b, t + 32);
  __builtin_amdgcn_sched_barrier(0);
  seq_add32(s, a);
  __builtin_amdgcn_sched_barrier(0);
  lds_load32(a, t + 64);
  __builtin_amdgcn_sched_barrier(0);
  seq_add32(s, b);
  __builtin_amdgcn_sched_barrier(0);
  seq_add32(s, a);
  return s;
}
constexpr int SEQ_NS = 8, SEQ_NC = 64, SEQ_LEN = 768 / SEQ_NS;
constexpr int SEQ_TAB_STRIDE = 12;                         // floats per candidate row (bank spread)
constexpr int SEQ_TAB_RESULT = SEQ_NC * SEQ_TAB_STRIDE;    // the sum, handed to every wave
constexpr int SEQ_TAB_FLOATS = SEQ_TAB_RESULT + 4;
// WALK: 1 if the calling wave is wave 0, 0 if it is not, 2 if that is known only
// at run time (a wave that cannot be wave 0 carries none of the walk's code).
template <int WALK>
__device__ __forceinline__ float seq_sum768_wg(const float* t, float* tab) {
  const int lane = (int)(threadIdx.x & 63), wave = (int)(threadIdx.x >> 6);
  // 1. binary64 prefix sums
  double p;
  {
    const f4 a = *(const f4*)(t + 12 * lane), b = *(const f4*)(t + 12 * lane + 4), c = *(const f4*)(t + 12 * lane + 8);
    p = (((double)a.x + (double)a.y) + ((double)a.z + (double)a.w)) +
        (((double)b.x + (double)b.y) + ((double)b.z + (double)b.w)) +
        (((double)c.x + (double)c.y) + ((double)c.z + (double)c.w));
  }
  p = p + dpp_d0<0x111, 0xf>(p);  // row_shr:1
  p = p + dpp_d0<0x112, 0xf>(p);  // row_shr:2
  p = p + dpp_d0<0x114, 0xf>(p);  // row_shr:4
  p = p + dpp_d0<0x118, 0xf>(p);  // row_shr:8
  p = p + dpp_d0<DPP_ROW_BCAST15, 0xa>(p);
  p = p + dpp_d0<DPP_ROW_BCAST31, 0xc>(p);
  const int ebits = __float_as_int((float)p);  // lane i: prefix through t[12i+11]
  // 2. candidate chains: segment k = wave starts after lane 8k-1's prefix
  {
    const int ek = wave == 0 ? 0 : f_ord(__builtin_amdgcn_readlane(ebits, 8 * wave - 1));
    const float start = __int_as_float(f_from_ord(ek + lane - SEQ_NC / 2));
    tab[lane * SEQ_TAB_STRIDE + wave] = seq_chain96(start, t + SEQ_LEN * wave);
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // 3. the walk, by wave 0 alone (its steps are scalar instructions, which the
  // waves of a compute unit would otherwise queue for), then handed to every wave
  // through LDS.
  if (WALK == 1 || (WALK == 2 && wave == 0)) {
    f4 tv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) tv[i] = *(const f4*)(tab + lane * SEQ_TAB_STRIDE + 4 * i);
    // Step k names the candidate whose start is the running sum S: with E the
    // estimate, its index is ord(S) - ord(E) + 32.  When S and E have the same
    // sign that is (bits(S) - bits(E)) + 32, or (bits(E) - bits(S)) + 32 for
    // negative E, i.e. (bits(S) ^ m) - c with m = 0 or ~0 by the sign of E and c
    // from E; an S of the other sign gives an index far out of range (the running
    // sum is never -0) and counts as a miss.  All of it in wrapping 32-bit
    // arithmetic.
    uint32_t sm[SEQ_NS], sc[SEQ_NS];
#pragma unroll
    for (int k = 0; k < SEQ_NS; ++k) {
      const int eb = k == 0 ? 0 : __builtin_amdgcn_readlane(ebits, 8 * k - 1);
      sm[k] = eb < 0 ? 0xffffffffu : 0u;
      sc[k] = eb < 0 ? ~((uint32_t)eb + (uint32_t)(SEQ_NC / 2)) : (uint32_t)eb - (uint32_t)(SEQ_NC / 2);
      asm volatile("" : "+s"(sm[k]), "+s"(sc[k]));  // formed before the walk, not inside its steps
    }
    // The steps run straight through with no branch (an index out of range is only
    // recorded); if one was out of range, the walk runs again, and a miss there runs
    // the segment's chain in place.
    uint32_t sb = 0, seen = 0;
#pragma unroll
    for (int k = 0; k < SEQ_NS; ++k) {
      const uint32_t dd = (sb ^ sm[k]) - sc[k];
      seen |= dd;  // >= SEQ_NC iff some step's index was out of range
      sb = (uint32_t)__builtin_amdgcn_readlane(__float_as_int(tv[k / 4][k % 4]), (int)(dd & (SEQ_NC - 1)));
    }
    if (__builtin_expect(seen >= (uint32_t)SEQ_NC, 0)) {
      sb = 0;
#pragma unroll
      for (int k = 0; k < SEQ_NS; ++k) {
        const uint32_t dd = (sb ^ sm[k]) - sc[k];
        if (dd < (uint32_t)SEQ_NC)
          sb = (uint32_t)__builtin_amdgcn_readlane(__float_as_int(tv[k / 4][k % 4]), (int)dd);
        else
          sb = (uint32_t)__builtin_amdgcn_readfirstlane(
              __float_as_int(seq_chain96(__uint_as_float(sb), t + SEQ_LEN * k)));
      }
    }
    if (lane == 0) tab[SEQ_TAB_RESULT] = __uint_as_float(sb);
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  return tab[SEQ_TAB_RESULT];
}

// The group-64 quantizer of quant_lane on a group held as 16 float4 by the 16
// lanes of a DPP row (thread T holds elements 4T..4T+3, group T/16): the same
// maximum (exact), scale m/127 and codes; codes go to xc[4T..4T+3], the scale of
// group g to xsc[g].
__device__ __forceinline__ int quant_code(float x, float s) {
  float q = rintf(x / s);
  if (q != q) q = 0.0f;
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return (int)q;
}
__device__ __forceinline__ void quant_frag16(const f4 y, int8_t* xc, float* xsc, int T) {
  float m = fmaxf(fmaxf(fabsf(y.x), fabsf(y.y)), fmaxf(fabsf(y.z), fabsf(y.w)));
  m = fmaxf(m, dpp_f<DPP_QUAD_1032>(m));
  m = fmaxf(m, dpp_f<DPP_QUAD_2301>(m));
  m = fmaxf(m, dpp_f<DPP_ROW_HALF_MIRROR>(m));
  m = fmaxf(m, dpp_f<DPP_ROW_MIRROR>(m));
  int packed = 0;
  float s = 0.0f;
  if (m != 0.0f) {
    s = m / 127.0f;
    packed = (quant_code(y.x, s) & 0xff) | (quant_code(y.y, s) & 0xff) << 8 | (quant_code(y.z, s) & 0xff) << 16 |
             (quant_code(y.w, s) & 0xff) << 24;
  }
  *(int*)(xc + 4 * T) = packed;
  if ((T & 15) == 0) xsc[T >> 4] = s;
}

// The sequential-order LayerNorm defined above, by all 512 threads of a workgroup,
// with both sums taken by seq_sum768_wg: the sequential loop's output bits.  xs, ys (LDS, distinct),
// tmp (768 floats) and tab of LDS scratch.  ys is complete for the
// workgroup after the caller's next barrier.  tab: SEQ_TAB_FLOATS floats.  WALK as
// for seq_sum768_wg.  With xc given, the output is also quantized in groups of 64
// (quant_frag16): codes into xc[0..767], scales into xsc[0..11].
template <int WALK>
__device__ __forceinline__ void layernorm_seq_wg(const float* xs, const float* __restrict__ gamma,
                                                 const float* __restrict__ beta, float* ys, float* tmp, float* tab,
                                                 int8_t* xc = nullptr, float* xsc = nullptr) {
  const float mean = seq_sum768_wg<WALK>(xs, tab) / 768.0f;
  const int T = (int)threadIdx.x;
  f4 d = {0.0f, 0.0f, 0.0f, 0.0f};
  if (T < 192) {
    d = *(const f4*)(xs + 4 * T) - mean;
    *(f4*)(tmp + 4 * T) = d * d;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  const float var = seq_sum768_wg<WALK>(tmp, tab) / 768.0f;
  const float r = 1.0f / sqrtf(var + 1e-5f);
  if (T < 192) {
    const f4 y = (d * r) * *(const f4*)(gamma + 4 * T) + *(const f4*)(beta + 4 * T);
    *(f4*)(ys + 4 * T) = y;
    if (xc) quant_frag16(y, xc, xsc, T);
  }
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not
// for its outstanding global loads and stores (a __syncthreads would also wait for
// every store of the wave to be acknowledged).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// This wave's LDS writes are complete before its later LDS reads (of other lanes' words).
__device__ __forceinline__ void wave_lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// ---- attention (one session, one head) --------------------------------------
// fp32 path, npos keys (1..128):
//   P_t,r = ((a.x + a.y) + (a.z + a.w)) with a = the float4 fmaf chain over i = 0..3
//     ascending of q[16r+4i..] * K_t[16r+4i..] (quarter r of the 64 dims);
//   s_t = ((P_t,0 + P_t,1) + (P_t,2 + P_t,3)) * 0.125   (1/sqrt(64));
//   m = max_t s_t;  e_t = exp_f32(s_t - m);
//   Z = Z_0 + Z_1 with Z_w = wave_sum of e_t over t in [64w, 64w+64);
//   w_t = e_t * rcp(Z) (the hardware reciprocal);
//   p_b = the fmaf chain over t in [8b, 8b+8), t < npos, ascending, of w_t*V_t,d (b < 16);
//   a_d = ((((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7))) + (((p8+p9)+(p10+p11))+((p12+p13)+(p14+p15)))).
// Every value is the same for a block of 128, 256 or 512 threads (the work is dealt
// out in fixed units).
constexpr int ATT_VB = 16;  // key blocks of the weighted sum
struct AttnSmem {
  float k[PMAX][DH + 4];  // padded rows, 16-byte aligned
  float v[PMAX][DH];
  float q[DH];
  float w[PMAX];          // scores, then weights
  float red[4];
  float part[ATT_VB][DH];  // per key-block partial outputs
};

// Stage key/value rows j0..j1-1 of one head into LDS with threads tid0..tid0+nthr-1
// of the block.  Row j of the keys is at kv(j) (64 keys), its values at kv(j) + D.
// UB > 1: a thread's loads of UB chunks are all in flight before their stores (a
// pass past the last chunk re-reads it and does not store it), so a few threads
// staging many rows pay one memory latency per UB chunks instead of one per chunk.
template <int UB = 1, class RowPtr>
__device__ __forceinline__ void attn_stage_rows(AttnSmem& sm, RowPtr kv, int j0, int j1, int tid0, int nthr) {
  const int t = (int)threadIdx.x - tid0;
  if (t < 0 || t >= nthr) return;
  const int n = (j1 - j0) * 16;
  if constexpr (UB == 1) {
    for (int idx = t; idx < n; idx += nthr) {
      const int j = j0 + (idx >> 4), c = (idx & 15) * 4;
      const float* row = kv(j);
      *(f4*)&sm.k[j][c] = *(const f4*)(row + c);
      *(f4*)&sm.v[j][c] = *(const f4*)(row + D + c);
    }
  } else {
    for (int base = t; base < n; base += UB * nthr) {
      f4 kk[UB], vv[UB];
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int idx = min(base + u * nthr, n - 1);
        const float* row = kv(j0 + (idx >> 4)) + (idx & 15) * 4;
        kk[u] = *(const f4*)row;
        vv[u] = *(const f4*)(row + D);
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int idx = base + u * nthr;
        if (idx < n) {
          const int j = j0 + (idx >> 4), c = (idx & 15) * 4;
          *(f4*)&sm.k[j][c] = kk[u];
          *(f4*)&sm.v[j][c] = vv[u];
        }
      }
    }
  }
}

// Stage all npos rows and the query with the first nthr threads, four chunks a pass.
template <class RowPtr>
__device__ __forceinline__ void attn_stage(AttnSmem& sm, RowPtr kv, int npos, const float* q, int nthr = 128) {
  attn_stage_rows<4>(sm, kv, 0, npos, 0, nthr);
  if (threadIdx.x < DH) sm.q[threadIdx.x] = q[threadIdx.x];
}

// Returns a_d in threads 0..63 (d = thread index); other threads return 0.  Every
// thread of the block (NTHR threads: 128, 256 or 512) must call it; it
// synchronises the block through LDS-only barriers.
template <int NTHR>
__device__ __forceinline__ float attn_compute(AttnSmem& sm, int npos) {
  static_assert(NTHR == 128 || NTHR == 256 || NTHR == 512, "key blocks are dealt out two per wave per pass");
  constexpr int nthr = NTHR;
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  // scores: unit u = 4*key + quarter, a lane quad per key
  for (int u = t; u < 4 * PMAX; u += nthr) {
    const int key = u >> 2, r = u & 3;
    f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f4 kr = *(const f4*)&sm.k[key][16 * r + 4 * i];
      const f4 qq = *(const f4*)&sm.q[16 * r + 4 * i];
      acc.x = fmaf(qq.x, kr.x, acc.x);
      acc.y = fmaf(qq.y, kr.y, acc.y);
      acc.z = fmaf(qq.z, kr.z, acc.z);
      acc.w = fmaf(qq.w, kr.w, acc.w);
    }
    float P = (acc.x + acc.y) + (acc.z + acc.w);
    P = P + dpp_f<DPP_QUAD_1032>(P);
    P = P + dpp_f<DPP_QUAD_2301>(P);
    if (r == 0 && key < npos) sm.w[key] = P * 0.125f;
  }
  lds_barrier();
  // Softmax by wave 0 alone over both halves of the 128 score slots: the maximum is
  // the fmaxf of the two wave maxima over slots 0..63 and 64..127, and Z the sum of
  // the two wave sums, the same trees and order as with one wave per half, so no
  // other wave takes part and no exchange between waves is needed.
  if (wv == 0) {
    const float s0 = lane < npos ? sm.w[lane] : -INFINITY;
    const float s1 = 64 + lane < npos ? sm.w[64 + lane] : -INFINITY;
    const float m = fmaxf(wave_max(s0), wave_max(s1));
    const float e0 = lane < npos ? exp_f32(s0 - m) : 0.0f;
    const float e1 = 64 + lane < npos ? exp_f32(s1 - m) : 0.0f;
    const float Z = wave_sum(e0) + wave_sum(e1);
    const float rz = __builtin_amdgcn_rcpf(Z);  // Z >= 1 (the maximum's term is 1)
    sm.w[lane] = e0 * rz;
    sm.w[64 + lane] = e1 * rz;
  }
  lds_barrier();
  // Two key blocks per pass (b0 and b0 + nw), their 32 LDS reads issued before the
  // two chains; a key past npos is skipped (its row holds no value of this step).
  constexpr int nw = NTHR / 64;
  for (int b0 = wv; b0 < ATT_VB; b0 += 2 * nw) {
    const int b1 = b0 + nw;
    const int n0 = min(max(npos - 8 * b0, 0), 8), n1 = min(max(npos - 8 * b1, 0), 8);
    float w0[8], v0[8], w1[8], v1[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      w0[jj] = sm.w[8 * b0 + jj];
      v0[jj] = sm.v[8 * b0 + jj][lane];
      w1[jj] = sm.w[8 * b1 + jj];
      v1[jj] = sm.v[8 * b1 + jj][lane];
    }
    float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (jj < n0) p0 = fmaf(w0[jj], v0[jj], p0);
      if (jj < n1) p1 = fmaf(w1[jj], v1[jj], p1);
    }
    sm.part[b0][lane] = p0;
    sm.part[b1][lane] = p1;
  }
  lds_barrier();
  float acc = 0.0f;
  if (wv == 0) {
    float p[ATT_VB];
#pragma unroll
    for (int b = 0; b < ATT_VB; ++b) p[b] = sm.part[b][lane];
#pragma unroll
    for (int w2 = 1; w2 < ATT_VB; w2 *= 2)
#pragma unroll
      for (int b = 0; b < ATT_VB; b += 2 * w2) p[b] = p[b] + p[b + w2];
    acc = p[0];
  }
  return acc;
}

// ---- the int8 path's attention, in the oracle's order -------------------------
// Its output is quantized, so it must not depend on a reduction tree:
//   s_t = (((0 + q_0*K_t,0) + q_1*K_t,1) + ... + q_63*K_t,63) * 0.125;  m = max_t s_t;
//   e_t = exp_spec(s_t - m);  Z = ((0 + e_0) + e_1) + ... ;  w_t = e_t / Z;
//   a_d = ((0 + w_0*V_0,d) + w_1*V_1,d) + ... .
// s + t[0] + ... + t[31] in order (t in LDS, 32 values in flight).
__device__ __forceinline__ float seq_chain32(float s, const float* t) {
  f4 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = *(const f4*)(t + 4 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = *(const f4*)(t + 16 + 4 * i);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) { s = s + a[i].x; s = s + a[i].y; s = s + a[i].z; s = s + a[i].w; }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) { s = s + b[i].x; s = s + b[i].y; s = s + b[i].z; s = s + b[i].w; }
  return s;
}
// binary64 inclusive prefix sum over the 64 lanes
__device__ __forceinline__ double wave_scan_d(double p) {
  p = p + dpp_d0<0x111, 0xf>(p);  // row_shr:1
  p = p + dpp_d0<0x112, 0xf>(p);  // row_shr:2
  p = p + dpp_d0<0x114, 0xf>(p);  // row_shr:4
  p = p + dpp_d0<0x118, 0xf>(p);  // row_shr:8
  p = p + dpp_d0<DPP_ROW_BCAST15, 0xa>(p);
  p = p + dpp_d0<DPP_ROW_BCAST31, 0xc>(p);
  return p;
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, l), hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (uint32_t)lo);
}
// Z = ((0 + w[0]) + w[1]) + ... + w[127] for nonnegative w (LDS; w[64j + lane] = e_j in
// the calling wave), by one wave, bit for bit the loop: lane 16k + c runs segment k
// (w[32k..32k+31]) from the binary32 value c - 8 steps away from the binary64 prefix
// estimate E_k of its start (nonnegative values order as their bit patterns), then a
// walk over the four segments takes the chain that started at the true running sum.
// The walk has no branches; if a true start lies outside its segment's candidates the
// walk runs again, taking such a segment's chain from the running sum itself.
__device__ __forceinline__ float seq_sum128_pos(const float* w, float e0, float e1) {
  const int lane = (int)(threadIdx.x & 63);
  const double p0 = wave_scan_d((double)e0), p1 = wave_scan_d((double)e1);
  const double h0 = readlane_d(p0, 31), t0 = readlane_d(p0, 63), h1 = readlane_d(p1, 31);
  const int eb1 = __float_as_int((float)h0), eb2 = __float_as_int((float)t0), eb3 = __float_as_int((float)(t0 + h1));
  const int k = lane >> 4, c = lane & 15;
  const int ek = k == 0 ? 0 : k == 1 ? eb1 : k == 2 ? eb2 : eb3;
  const float res = seq_chain32(__int_as_float(ek + c - 8), w + 32 * k);
  const uint32_t eb[4] = {0u, (uint32_t)eb1, (uint32_t)eb2, (uint32_t)eb3};
  uint32_t sb = 0, miss = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t dd = sb - eb[s] + 8u;
    miss |= (uint32_t)(dd >= 16u);
    sb = (uint32_t)__builtin_amdgcn_readlane(__float_as_int(res), 16 * s + (int)(dd & 15u));
  }
  if (__builtin_expect(miss != 0, 0)) {
    sb = 0;
#pragma unroll 1
    for (int s = 0; s < 4; ++s) {
      const uint32_t dd = sb - eb[s] + 8u;
      if (dd < 16u)
        sb = (uint32_t)__builtin_amdgcn_readlane(__float_as_int(res), 16 * s + (int)dd);
      else
        sb = (uint32_t)__builtin_amdgcn_readfirstlane(__float_as_int(seq_chain32(__uint_as_float(sb), w + 32 * s)));
    }
  }
  return __uint_as_float(sb);
}
// Threads t < npos score key t (threads 0..127: at least two waves); after one LDS
// barrier wave 0 alone takes the softmax, Z, the weights and the ordered weighted
// sums.  Returns a_d in the threads of wave 0 (d = lane), 0 elsewhere.  Every thread
// of the block (128 or more) must call it.  sm.w is overwritten; the caller
// synchronises before sm is written again.
__device__ __forceinline__ float attn_compute_seq(AttnSmem& sm, int npos) {
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  if (t < PMAX) {
    float s = -INFINITY;
    if (t < npos) {
      // 16 key and query values in flight while the previous 16 are added
      float acc = 0.0f;
      f4 ka[4], qa[4], kb[4], qb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ka[i] = *(const f4*)&sm.k[t][4 * i];
        qa[i] = *(const f4*)&sm.q[4 * i];
      }
#pragma unroll
      for (int bb = 0; bb < 4; bb += 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kb[i] = *(const f4*)&sm.k[t][16 * (bb + 1) + 4 * i];
          qb[i] = *(const f4*)&sm.q[16 * (bb + 1) + 4 * i];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc = acc + qa[i].x * ka[i].x;
          acc = acc + qa[i].y * ka[i].y;
          acc = acc + qa[i].z * ka[i].z;
          acc = acc + qa[i].w * ka[i].w;
        }
        if (bb + 2 < 4) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            ka[i] = *(const f4*)&sm.k[t][16 * (bb + 2) + 4 * i];
            qa[i] = *(const f4*)&sm.q[16 * (bb + 2) + 4 * i];
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc = acc + qb[i].x * kb[i].x;
          acc = acc + qb[i].y * kb[i].y;
          acc = acc + qb[i].z * kb[i].z;
          acc = acc + qb[i].w * kb[i].w;
        }
      }
      s = acc * 0.125f;
    }
    sm.w[t] = s;
  }
  lds_barrier();
  if (wv != 0) return 0.0f;
  const float s0 = sm.w[lane], s1 = sm.w[64 + lane];
  const float m = fmaxf(wave_max(s0), wave_max(s1));
  const float e0 = lane < npos ? exp_spec(s0 - m) : 0.0f;
  const float e1 = 64 + lane < npos ? exp_spec(s1 - m) : 0.0f;
  sm.w[lane] = e0;
  sm.w[64 + lane] = e1;
  wave_lds_wait();
  float Z;
  if (npos <= 48) {
    // the slots past npos hold +0, which leaves a nonnegative running sum unchanged
    Z = 0.0f;
    for (int j = 0; j < npos; j += 8) {
      const f4 a = *(const f4*)&sm.w[j], b = *(const f4*)&sm.w[j + 4];
      Z = Z + a.x; Z = Z + a.y; Z = Z + a.z; Z = Z + a.w;
      Z = Z + b.x; Z = Z + b.y; Z = Z + b.z; Z = Z + b.w;
    }
  } else {
    Z = seq_sum128_pos(sm.w, e0, e1);
  }
  sm.w[lane] = e0 / Z;
  sm.w[64 + lane] = e1 / Z;
  wave_lds_wait();
  float acc = 0.0f;
  int j = 0;
  for (; j + 8 <= npos; j += 8) {
    const f4 wa = *(const f4*)&sm.w[j], wb = *(const f4*)&sm.w[j + 4];
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = sm.v[j + u][lane];
    acc = acc + wa.x * v[0]; acc = acc + wa.y * v[1]; acc = acc + wa.z * v[2]; acc = acc + wa.w * v[3];
    acc = acc + wb.x * v[4]; acc = acc + wb.y * v[5]; acc = acc + wb.z * v[6]; acc = acc + wb.w * v[7];
  }
  for (; j < npos; ++j) acc = acc + sm.w[j] * sm.v[j][lane];
  return acc;
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
  return quant_code(x, s);
}

// One output of an int8 group-64 projection with K inputs.  Lane l holds the row's
// codes at bytes 1024*i + 16*l (i < NCH), i.e. group 16*i + l/4; swl is lane g's
// weight scale for group g (g < K/64).  xc/xsc are the input codes and scales.
//   acc[g] = sum of the 64 code products of group g (v_dot4, then two exact integer
//   quad_sum steps inside each 4-lane quad), moved to lane g;
//   t[g] = ((float)acc[g] * sw[g]) * sx[g] in lane g;
//   y = 0; y = y + t[g] for g = 0..K/64-1  (fixed order, through readlane).
// cap_acc (may be null) receives acc[0..K/64-1].  Bias excluded.
// q8_group_acc alone: acc[lane] in lane < K/64 (lane = lane_id()).
template <int K>
__device__ __forceinline__ int q8_group_acc(const i4 (&wc)[(K + 1023) / 1024], const int8_t* xc, int lane) {
  constexpr int NCH = (K + 1023) / 1024;
  int accg = 0;  // acc[lane] for lane < G
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int off = 1024 * i + 16 * lane;
    int p = 0;
    if (off < K) {
      const i4 xv = *(const i4*)(xc + off);
      p = __builtin_amdgcn_sdot4(wc[i].x, xv.x, p, false);
      p = __builtin_amdgcn_sdot4(wc[i].y, xv.y, p, false);
      p = __builtin_amdgcn_sdot4(wc[i].z, xv.z, p, false);
      p = __builtin_amdgcn_sdot4(wc[i].w, xv.w, p, false);
    }
    p = quad_sum(p);
    const int gi = __shfl(p, 4 * (lane & 15));  // group 16*i + (lane & 15)
    if ((lane >> 4) == i) accg = gi;
  }
  return accg;
}
template <int K>
__device__ __forceinline__ float q8_dot(const i4 (&wc)[(K + 1023) / 1024], float swl, const int8_t* xc,
                                        const float* xsc, int32_t* cap_acc) {
  constexpr int G = K / 64;
  const int lane = lane_id();
  const int accg = q8_group_acc<K>(wc, xc, lane);
  if (cap_acc && lane < G) cap_acc[lane] = accg;
  const float t = lane < G ? ((float)accg * swl) * xsc[lane] : 0.0f;
  float y = 0.0f;
#pragma unroll
  for (int g = 0; g < G; ++g) y = y + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), g));
  return y;
}

// The 768-input form of q8_dot with the weight scales in quad layout: lane l < 48
// holds the row's codes at bytes 16l..16l+15 (group g = l/4) and swq, the row's
// scale of group l/4 (lanes 48..63: any values, they contribute no term).  acc[g] is the exact
// quad sum in lanes 4g..4g+3, so t[g] is formed there and the fixed-order rescale
// reads lane 4g: the same values and operations as q8_dot<768>, without moving the
// group sums across lanes first.  cap_acc as for q8_dot.
__device__ __forceinline__ float q8_dot768q(const i4 wc, float swq, const int8_t* xc, const float* xsc,
                                            int32_t* cap_acc) {
  const int lane = lane_id();
  const i4 xv = *(const i4*)(xc + 16 * min(lane, 47));
  int p = 0;
  p = __builtin_amdgcn_sdot4(wc.x, xv.x, p, false);
  p = __builtin_amdgcn_sdot4(wc.y, xv.y, p, false);
  p = __builtin_amdgcn_sdot4(wc.z, xv.z, p, false);
  p = __builtin_amdgcn_sdot4(wc.w, xv.w, p, false);
  p = quad_sum(p);
  if (cap_acc && lane < 48 && (lane & 3) == 0) cap_acc[lane >> 2] = p;
  const float t = lane < 48 ? ((float)p * swq) * xsc[min(lane >> 2, 11)] : 0.0f;
  float y = 0.0f;
#pragma unroll
  for (int g = 0; g < 12; ++g) y = y + __int_as_float(__builtin_amdgcn_readlane(__float_as_int(t), 4 * g));
  return y;
}
// Four int8 rows in quad layout evaluated together, each to q8_dot768q's value.
// The exact group accumulators are summed over each quad transposed (partners
// lane^1 then lane^2, each lane keeping one of the rows it shares with its partner),
// so lane 4g + i holds row i's accumulator of group g; its term is
// t = ((float)acc * sw_i) * sx_g, and the twelve ordered adds
// y = ((0 + t_0) + t_1) + ... + t_11 run once for the four rows, lane i of row 0
// taking t_g from lane 4g + i (a row shift inside rows 0..2 of the wave, those rows
// first moved to row 0).  Lanes 0..3 return rows 0..3; other lanes, any value.
// cap_acc[i] (or null) receives row i's twelve group accumulators.
template <int CTRL>
__device__ __forceinline__ float dpp_add_f(float y, float t) {
  return dpp_f<CTRL>(t) + y;  // t + y == y + t exactly
}
__device__ __forceinline__ float q8_dot768q_x4(const i4 (&wc)[4], const float (&swq)[4], const int8_t* xc,
                                               const float* xsc, int32_t* const (&cap_acc)[4]) {
  const int lane = lane_id();
  const i4 xv = *(const i4*)(xc + 16 * min(lane, 47));
  int p[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int a = 0;
    a = __builtin_amdgcn_sdot4(wc[k].x, xv.x, a, false);
    a = __builtin_amdgcn_sdot4(wc[k].y, xv.y, a, false);
    a = __builtin_amdgcn_sdot4(wc[k].z, xv.z, a, false);
    a = __builtin_amdgcn_sdot4(wc[k].w, xv.w, a, false);
    p[k] = a;
  }
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
  const int a0 = (b0 ? p[1] : p[0]) + dpp_i<DPP_QUAD_1032>(b0 ? p[0] : p[1]);  // row b0
  const int a1 = (b0 ? p[3] : p[2]) + dpp_i<DPP_QUAD_1032>(b0 ? p[2] : p[3]);  // row 2 + b0
  const int acc = (b1 ? a1 : a0) + dpp_i<DPP_QUAD_2301>(b1 ? a0 : a1);         // row lane & 3
  const int i = lane & 3;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (cap_acc[k] && lane < 48 && i == k) cap_acc[k][lane >> 2] = acc;
  // the lane's row scale by selects on register values (an indexed read of swq would
  // put the caller's registers in scratch memory)
  float sv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    sv[k] = swq[k];
    asm volatile("" : "+v"(sv[k]));
  }
  const float sw = i == 0 ? sv[0] : i == 1 ? sv[1] : i == 2 ? sv[2] : sv[3];
  const float t = lane < 48 ? ((float)acc * sw) * xsc[min(lane >> 2, 11)] : 0.0f;
  const float t1 = row1_to_row0(t), t2 = row2_to_row0(t);
  float y = 0.0f + t;
  y = dpp_add_f<DPP_ROW_SL4>(y, t);
  y = dpp_add_f<DPP_ROW_SL8>(y, t);
  y = dpp_add_f<DPP_ROW_SL12>(y, t);
  y = y + t1;
  y = dpp_add_f<DPP_ROW_SL4>(y, t1);
  y = dpp_add_f<DPP_ROW_SL8>(y, t1);
  y = dpp_add_f<DPP_ROW_SL12>(y, t1);
  y = y + t2;
  y = dpp_add_f<DPP_ROW_SL4>(y, t2);
  y = dpp_add_f<DPP_ROW_SL8>(y, t2);
  y = dpp_add_f<DPP_ROW_SL12>(y, t2);
  return y;
}

// Codes of int8 row r of a [rows][768] matrix and its group scales in quad layout,
// for q8_dot768q (nontemporal loads).  Lanes 48..63 hold copies of lane 47's codes
// and scale: q8_dot768q takes no term from those lanes, so nothing here uses the
// loaded values and the loads stay in flight until the dot reads them.
__device__ __forceinline__ void q8_load_row768q(i4& wc, float& swq, const int8_t* codes, const float* scales, int r) {
  const int lane = lane_id_fresh();
  wc = __builtin_nontemporal_load((const i4*)(codes + (size_t)r * 768 + 16 * min(lane, 47)));
  swq = scales[(size_t)r * 12 + min(lane >> 2, 11)];
}

// Load the codes and lane-g scale of int8 row r of a [rows][K] matrix (nontemporal).
template <int K>
__device__ __forceinline__ void q8_load_row(i4 (&wc)[(K + 1023) / 1024], float& swl, const int8_t* codes,
                                            const float* scales, int r) {
  constexpr int NCH = (K + 1023) / 1024, G = K / 64;
  const int lane = lane_id_fresh();
  const int8_t* row = codes + (size_t)r * K;
  // every lane loads (lanes past the row re-read its last 16 bytes), so callers can
  // keep an identical memory-instruction stream on every path
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int off = 1024 * i + 16 * lane;
    const i4 v = __builtin_nontemporal_load((const i4*)(row + min(off, K - 16)));
    wc[i] = off < K ? v : i4{0, 0, 0, 0};
  }
  const float sv = scales[(size_t)r * G + min(lane, G - 1)];
  swl = lane < G ? sv : 0.0f;
}

}  // namespace g2
