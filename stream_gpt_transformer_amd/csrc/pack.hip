// One-time packing of the checkpoint into the device layout (gpt2.s page, weight
// tiling paragraph: the program re-lays the [input][output] block matrices once at
// startup so the matrix kernel streams them in order; here the re-layout is to
// [output][input] rows for wavefront-wide coalesced row reads), int8 group-64
// quantization of the projection weights (marXiv 2609.00018 abstract), and the
// binary16 storage form (gpt2.s page, options: weights kept as half precision and
// widened to binary32 for the arithmetic).
#include <hip/hip_fp16.h>

#include "device.hpp"
#include "internal.hpp"

namespace g2 {

// dst[N][K] = transpose of src[K][N]; 64x64 tiles through LDS, both sides coalesced.
__global__ __launch_bounds__(256) void k_transpose(const float* __restrict__ src, float* __restrict__ dst,
                                                   int K, int N) {
  __shared__ float tile[64][65];
  const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int kk = i >> 6, nn = i & 63;
    tile[kk][nn] = src[(size_t)(k0 + kk) * N + n0 + nn];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int nn = i >> 6, kk = i & 63;
    dst[(size_t)(n0 + nn) * K + k0 + kk] = tile[kk][nn];
  }
}

// binary16 dst[N][K] of src[K][N] (round to nearest even, overflow to infinity).
__global__ __launch_bounds__(256) void k_transpose_f16(const float* __restrict__ src, uint16_t* __restrict__ dst,
                                                       int K, int N) {
  __shared__ float tile[64][65];
  const int n0 = blockIdx.x * 64, k0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int kk = i >> 6, nn = i & 63;
    tile[kk][nn] = src[(size_t)(k0 + kk) * N + n0 + nn];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int nn = i >> 6, kk = i & 63;
    dst[(size_t)(n0 + nn) * K + k0 + kk] = __half_as_ushort(__float2half_rn(tile[kk][nn]));
  }
}

// binary16 copy of n values (the token table).
__global__ __launch_bounds__(256) void k_to_f16(const float* __restrict__ src, uint16_t* __restrict__ dst, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = __half_as_ushort(__float2half_rn(src[i]));
}

// int8 codes [N][K] and scales [N][K/64] of a checkpoint matrix src[K][N]: group g of
// output n holds inputs 64g..64g+63 of column n.  Block = (64 outputs, one group).
__global__ __launch_bounds__(256) void k_quant_in_out(const float* __restrict__ src, int8_t* __restrict__ codes,
                                                      float* __restrict__ scales, int K, int N) {
  __shared__ float tile[64][65];
  const int n0 = blockIdx.x * 64, g = blockIdx.y, G = K / 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int kk = i >> 6, nn = i & 63;
    tile[kk][nn] = src[(size_t)(g * 64 + kk) * N + n0 + nn];
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int c = wave; c < 64; c += 4) {
    float s;
    const int code = quant_lane(tile[lane][c], s);
    codes[(size_t)(n0 + c) * K + g * 64 + lane] = (int8_t)code;
    if (lane == 0) scales[(size_t)(n0 + c) * G + g] = s;
  }
}

// int8 codes of rows already stored [rows][K] (the tied head: wte rows).
__global__ __launch_bounds__(256) void k_quant_rows(const float* __restrict__ src, int8_t* __restrict__ codes,
                                                    float* __restrict__ scales, int rows, int K) {
  const int G = K / 64;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (item >= rows * G) return;
  const int r = item / G, g = item % G;
  float s;
  const int code = quant_lane(src[(size_t)r * K + g * 64 + lane], s);
  codes[(size_t)r * K + g * 64 + lane] = (int8_t)code;
  if (lane == 0) scales[(size_t)r * G + g] = s;
}

// Weight-scale groups of gw inputs (gw a multiple of 64 dividing K; the marXiv
// 2609.00018 abstract's granularity variants): output n, group j of a checkpoint
// matrix src[K][N] gets scale (max |w| over the group)/127 and codes
// clamp(rint(w/scale), -127, 127) (0 for an all-zero group), as quant_lane does
// for 64 inputs.  The scale is written to each 64-input slot of the group, so the
// int8 kernels read one scale per 64 inputs whatever gw is.  Thread = (output n,
// group blockIdx.y); one-time work.
__global__ __launch_bounds__(256) void k_quant_in_out_g(const float* __restrict__ src, int8_t* __restrict__ codes,
                                                        float* __restrict__ scales, int K, int N, int gw) {
  const int n = blockIdx.x * 256 + threadIdx.x, j = blockIdx.y;
  if (n >= N) return;
  const float* col = src + (size_t)j * gw * N + n;
  float m = 0.0f;
  for (int i = 0; i < gw; ++i) m = fmaxf(m, fabsf(col[(size_t)i * N]));
  const float sc = m == 0.0f ? 0.0f : m / 127.0f;
  int8_t* c = codes + (size_t)n * K + (size_t)j * gw;
  for (int i = 0; i < gw; i += 4) {
    int packed = 0;
    if (m != 0.0f)
      for (int e = 0; e < 4; ++e) packed |= (quant_code(col[(size_t)(i + e) * N], sc) & 0xff) << (8 * e);
    *(int*)(c + i) = packed;
  }
  for (int t = 0; t < gw / 64; ++t) scales[(size_t)n * (K / 64) + (size_t)j * (gw / 64) + t] = sc;
}

// The same for rows already stored [rows][K] (the tied head: wte rows).  Thread =
// (row, group).
__global__ __launch_bounds__(256) void k_quant_rows_g(const float* __restrict__ src, int8_t* __restrict__ codes,
                                                      float* __restrict__ scales, int rows, int K, int gw) {
  const long long item = (long long)blockIdx.x * 256 + threadIdx.x;
  const int ng = K / gw;
  if (item >= (long long)rows * ng) return;
  const int r = (int)(item / ng), j = (int)(item % ng);
  const float* x = src + (size_t)r * K + (size_t)j * gw;
  float m = 0.0f;
  for (int i = 0; i < gw; ++i) m = fmaxf(m, fabsf(x[i]));
  const float sc = m == 0.0f ? 0.0f : m / 127.0f;
  int8_t* c = codes + (size_t)r * K + (size_t)j * gw;
  for (int i = 0; i < gw; i += 4) {
    int packed = 0;
    if (m != 0.0f)
      for (int e = 0; e < 4; ++e) packed |= (quant_code(x[i + e], sc) & 0xff) << (8 * e);
    *(int*)(c + i) = packed;
  }
  for (int t = 0; t < gw / 64; ++t) scales[(size_t)r * (K / 64) + (size_t)j * (gw / 64) + t] = sc;
}

// q8_group: the int8 weight-scale group (64, a larger multiple of 64 dividing 768,
// or 0 for one scale per output row).
hipError_t launch_pack(const float* ck_, char* packed, int flags, hipStream_t s, int q8_group) {
  const PackedLayout pl = packed_layout(flags);
  float* wte = (float*)(packed + pl.wte);
  float* wpe = (float*)(packed + pl.wpe);
  float* small = (float*)(packed + pl.small);
  hipError_t e;
  auto cp = [&](float* dst, size_t src_off, size_t n) {
    return hipMemcpyAsync(dst, ck_ + src_off, n * 4, hipMemcpyDeviceToDevice, s);
  };
  if ((e = cp(wte, ck::WTE, (size_t)V * D))) return e;
  if ((e = cp(wpe, ck::WPE, (size_t)PMAX * D))) return e;
  for (int l = 0; l < L; ++l) {
    const size_t b = ck::BLOCK0 + (size_t)l * ck::BLOCK;
    float* sl = small + (size_t)l * sp::PER_LAYER;
    if ((e = cp(sl + sp::LN1_G, b + ck::LN1_G, D))) return e;
    if ((e = cp(sl + sp::LN1_B, b + ck::LN1_B, D))) return e;
    if ((e = cp(sl + sp::B_QKV, b + ck::ATTN_B, D3))) return e;
    if ((e = cp(sl + sp::B_O, b + ck::APROJ_B, D))) return e;
    if ((e = cp(sl + sp::LN2_G, b + ck::LN2_G, D))) return e;
    if ((e = cp(sl + sp::LN2_B, b + ck::LN2_B, D))) return e;
    if ((e = cp(sl + sp::B_FC, b + ck::FC_B, F))) return e;
    if ((e = cp(sl + sp::B_PR, b + ck::MPROJ_B, D))) return e;
  }
  if ((e = cp(small + sp::LNF_G, ck::LNF_G, D))) return e;
  if ((e = cp(small + sp::LNF_B, ck::LNF_B, D))) return e;

  const size_t src_off[4] = {ck::ATTN_W, ck::APROJ_W, ck::FC_W, ck::MPROJ_W};
  for (int l = 0; l < L; ++l) {
    const size_t b = ck::BLOCK0 + (size_t)l * ck::BLOCK;
    for (int m = 0; m < 4; ++m) {
      const int K = mat_cols(m), N = mat_rows(m);
      const float* src = ck_ + b + src_off[m];
      if (flags & 1) {
        float* dst = (float*)(packed + pl.f32) + (size_t)l * LAYER_ELEMS + mat_elem_off(m);
        hipLaunchKernelGGL(k_transpose, dim3(N / 64, K / 64), dim3(256), 0, s, src, dst, K, N);
      }
      if (flags & 4) {
        uint16_t* dst = (uint16_t*)(packed + pl.f16) + (size_t)l * LAYER_ELEMS + mat_elem_off(m);
        hipLaunchKernelGGL(k_transpose_f16, dim3(N / 64, K / 64), dim3(256), 0, s, src, dst, K, N);
      }
      if (flags & 2) {
        int8_t* codes = (int8_t*)(packed + pl.q8_codes) + (size_t)l * LAYER_ELEMS + mat_elem_off(m);
        float* scales = (float*)(packed + pl.q8_scales) + (size_t)l * LAYER_SCALES + mat_scale_off(m);
        if (q8_group == 64) {
          hipLaunchKernelGGL(k_quant_in_out, dim3(N / 64, K / 64), dim3(256), 0, s, src, codes, scales, K, N);
        } else {
          const int gw = q8_group == 0 ? K : q8_group;
          hipLaunchKernelGGL(k_quant_in_out_g, dim3((N + 255) / 256, K / gw), dim3(256), 0, s, src, codes, scales,
                             K, N, gw);
        }
      }
    }
  }
  if (flags & 4) {
    const size_t n = (size_t)V * D;
    hipLaunchKernelGGL(k_to_f16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ck_ + ck::WTE,
                       (uint16_t*)(packed + pl.f16) + (size_t)L * LAYER_ELEMS, n);
  }
  if (flags & 2) {
    int8_t* codes = (int8_t*)(packed + pl.q8_codes) + (size_t)L * LAYER_ELEMS;
    float* scales = (float*)(packed + pl.q8_scales) + (size_t)L * LAYER_SCALES;
    if (q8_group == 64) {
      const int items = V * (D / 64);
      hipLaunchKernelGGL(k_quant_rows, dim3((items + 3) / 4), dim3(256), 0, s, ck_ + ck::WTE, codes, scales, V, D);
    } else {
      const int gw = q8_group == 0 ? D : q8_group;
      const long long items = (long long)V * (D / gw);
      hipLaunchKernelGGL(k_quant_rows_g, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, ck_ + ck::WTE, codes,
                         scales, V, D, gw);
    }
  }
  return hipGetLastError();
}

}  // namespace g2
