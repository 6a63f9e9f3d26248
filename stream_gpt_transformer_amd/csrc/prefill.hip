// Full-prefix inference (LeanExe GPT-2 README, infer paragraph): 1..128 tokens run
// as row batches through the 12 blocks; only the final row reaches the tied head.
// The block projections are dense T x K by K x N contractions and run on the fp32
// matrix cores (v_mfma_f32_16x16x4_f32); LayerNorm, causal attention and the head
// reuse the decode building blocks.
#include "device.hpp"
#include "internal.hpp"

namespace g2 {

typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Epi { EPI_STORE = 0, EPI_RESID = 1, EPI_GELU = 2, EPI_PART = 3 };

// C = A[M][K] * W[N][K]^T (+ epilogue).  Block tile 64x64, four waves each owning a
// 32x32 quarter as 2x2 MFMA 16x16 tiles; K staged through LDS 32 at a time.
// MFMA 16x16x4 f32 operand layout: lane l supplies A[l%16][l/16] and B[l/16][l%16];
// result register r of lane l is C[4*(l/16) + r][l%16].
// EPI_PART writes raw partial sums of the K range [kbeg, kbeg+klen) to
// part[blockIdx.z][M][N] (split-K; the caller sums the parts in a fixed order).
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm(const float* __restrict__ A, int lda, const float* __restrict__ W,
                                              int K, int M, int N, const float* __restrict__ bias,
                                              float* __restrict__ C, int ldc, int klen) {
  __shared__ float As[64][33];
  __shared__ float Ws[64][33];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int kbeg = blockIdx.z * klen;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0, 0, 0, 0};
  for (int k0 = kbeg; k0 < kbeg + klen; k0 += 32) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int idx = threadIdx.x + 256 * it;
      const int r = idx >> 5, c = idx & 31;
      As[r][c] = m0 + r < M ? A[(size_t)(m0 + r) * lda + k0 + c] : 0.0f;
      Ws[r][c] = W[(size_t)(n0 + r) * K + k0 + c];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[32 * wm + 16 * i + (lane & 15)][4 * kk + (lane >> 4)];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = Ws[32 * wn + 16 * j + (lane & 15)][4 * kk + (lane >> 4)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 32 * wm + 16 * i + 4 * (lane >> 4) + r;
        const int col = n0 + 32 * wn + 16 * j + (lane & 15);
        if (row >= M) continue;
        const float v = acc[i][j][r];
        if constexpr (EPI == EPI_PART) {
          C[((size_t)blockIdx.z * M + row) * ldc + col] = v;
        } else {
          const float y = bias ? v + bias[col] : v;
          float* c = C + (size_t)row * ldc + col;
          if constexpr (EPI == EPI_STORE) *c = y;
          else if constexpr (EPI == EPI_RESID) *c = *c + y;
          else *c = gelu_tanh(y);
        }
      }
}

// x[t][n] += ((part0 + part1) + ... + part{S-1}) + bias  (fixed order).
__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ part, int S, int M, int N,
                                                      const float* __restrict__ bias, float* __restrict__ x) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * N) return;
  float v = part[i];
  for (int s = 1; s < S; ++s) v = v + part[(size_t)s * M * N + i];
  x[i] = x[i] + (v + bias[i % N]);
}

struct Toks {
  uint32_t t[PMAX];
};

__global__ __launch_bounds__(192) void k_pf_embed(const Weights w, const Toks tk, float* x) {
  const int t = blockIdx.x, i = threadIdx.x;
  const f4 e = *(const f4*)(w.wte + (size_t)tk.t[t] * D + 4 * i);
  const f4 p = *(const f4*)(w.wpe + (size_t)t * D + 4 * i);
  *(f4*)(x + (size_t)t * D + 4 * i) = e + p;
}

// One wave per row.
__global__ __launch_bounds__(64) void k_pf_ln(const float* __restrict__ x, const float* gamma, const float* beta,
                                              float* __restrict__ y) {
  f4 v[3];
  load_frag<3>(v, x + (size_t)blockIdx.x * D);
  layernorm_frag(v, gamma, beta);
  store_frag<3>(y + (size_t)blockIdx.x * D, v);
}

// Causal attention of head blockIdx.x for row blockIdx.y over rows 0..t of the
// row-batch QKV buffer.
__global__ __launch_bounds__(128) void k_pf_attn(const float* __restrict__ qkv, float* __restrict__ att) {
  __shared__ AttnSmem sm;
  const int h = blockIdx.x, t = blockIdx.y;
  auto kv = [&](int j) { return qkv + (size_t)j * D3 + D + h * DH; };
  attn_stage(sm, kv, t + 1, qkv + (size_t)t * D3 + h * DH);
  __syncthreads();
  const float o = attn_compute(sm, t + 1);
  if (threadIdx.x < DH) att[(size_t)t * D + h * DH + threadIdx.x] = o;
}

hipError_t launch_head_f32(const Weights& w, const float* x_row, float* logits, hipStream_t s);

template <int EPI>
static void gemm(const float* A, int lda, const float* W, int K, int M, int N, const float* bias, float* C,
                 int ldc, int split, hipStream_t s) {
  dim3 grid(N / 64, (M + 63) / 64, split);
  hipLaunchKernelGGL((k_gemm<EPI>), grid, dim3(256), 0, s, A, lda, W, K, M, N, bias, C, ldc, K / split);
}

hipError_t launch_infer(const Weights& w, const Work& k, const uint32_t* toks, int n, float* logits,
                        hipStream_t s) {
  Toks tk{};
  for (int t = 0; t < n; ++t) tk.t[t] = toks[t];
  hipLaunchKernelGGL(k_pf_embed, dim3(n), dim3(192), 0, s, w, tk, k.pf_x);
  for (int l = 0; l < L; ++l) {
    hipLaunchKernelGGL(k_pf_ln, dim3(n), dim3(64), 0, s, k.pf_x, small_p(w, l, sp::LN1_G), small_p(w, l, sp::LN1_B),
                       k.pf_h);
    gemm<EPI_STORE>(k.pf_h, D, f32_mat(w, l, M_QKV), D, n, D3, small_p(w, l, sp::B_QKV), k.pf_qkv, D3, 1, s);
    hipLaunchKernelGGL(k_pf_attn, dim3(H, n), dim3(128), 0, s, k.pf_qkv, k.pf_att);
    gemm<EPI_RESID>(k.pf_att, D, f32_mat(w, l, M_O), D, n, D, small_p(w, l, sp::B_O), k.pf_x, D, 1, s);
    hipLaunchKernelGGL(k_pf_ln, dim3(n), dim3(64), 0, s, k.pf_x, small_p(w, l, sp::LN2_G), small_p(w, l, sp::LN2_B),
                       k.pf_h);
    gemm<EPI_GELU>(k.pf_h, D, f32_mat(w, l, M_FC), D, n, F, small_p(w, l, sp::B_FC), k.pf_u, F, 1, s);
    gemm<EPI_PART>(k.pf_u, F, f32_mat(w, l, M_PR), F, n, D, nullptr, k.pf_part, D, PF_SPLIT, s);
    hipLaunchKernelGGL(k_split_reduce, dim3((n * D + 255) / 256), dim3(256), 0, s, k.pf_part, PF_SPLIT, n, D,
                       small_p(w, l, sp::B_PR), k.pf_x);
  }
  return launch_head_f32(w, k.pf_x + (size_t)(n - 1) * D, logits, s);
}

hipError_t launch_gemm_test(const float* A, const float* W, float* C, int M, int N, int K, hipStream_t s) {
  gemm<EPI_STORE>(A, K, W, K, M, N, nullptr, C, N, 1, s);
  return hipGetLastError();
}

}  // namespace g2
