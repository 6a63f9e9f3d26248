// Full-prefix inference (LeanExe GPT-2 README, infer paragraph): 1..128 tokens run
// as row batches through the 12 blocks; only the final row reaches the tied head.
//
// The block projections are dense T x K by K x N contractions on the fp32 matrix
// cores (v_mfma_f32_16x16x4_f32).  With T <= 128 rows every projection is short
// and wide, so each wavefront owns a 32 x 32 output tile over a slice of K and
// streams both operands straight from memory into registers, four 16-deep K steps
// ahead; the K dimension is split so that every projection launches about 200
// workgroups or fewer, one per compute unit.  The split partial sums are
// added in a fixed order by the kernel that applies the epilogue (bias, GELU,
// residual, and the LayerNorm that follows a residual), so results do not depend
// on timing.  Causal attention stages each head's key/value rows in LDS once per
// eight query rows.
#include "device.hpp"
#include "internal.hpp"

namespace g2 {

typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Epi { EPI_STORE = 0, EPI_PART = 1 };

// C = A[M][K] * W[N][K]^T over the K range [z*klen, (z+1)*klen) (z = blockIdx.y).
// Workgroup: 4 waves, wave w owns rows 32w..32w+31 and the workgroup's 32 columns
// n0 = 32*blockIdx.x.  Rows at or past M read row M-1 and store nothing.
// MFMA 16x16x4 f32 operand layout: lane l supplies A[l%16][kk] and B[kk][l%16]
// with kk = l/16; result register r of lane l is C[4*(l/16) + r][l%16].  Within a
// 16-wide K step, sub-step s feeds kk = l/16 the element k + 4*(l/16) + s to both
// operands, so each lane reads four consecutive K elements as one 16-byte load
// and the four sub-steps cover the step's 16 elements once each.
// PF steps are in flight per wave.  Every loop pass issues the same loads (past
// the last step they re-read it), so the compiler's wait counts stay exact and a
// wait never drains the prefetches behind it.
// EPI_STORE: C = acc + bias (bias may be null);
// EPI_PART: part[z][row][col] = acc (ldc = N).
template <int EPI, int PF>
__global__ __launch_bounds__(256) void k_mm(const float* __restrict__ A, int lda, const float* __restrict__ W,
                                           int ldw, int M, int N, const float* __restrict__ bias,
                                           float* __restrict__ C, int ldc, int klen) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m0 = 32 * wave;
  if (m0 >= M) return;
  const int n0 = 32 * blockIdx.x;
  const int kbeg = blockIdx.y * klen;
  const int r = lane & 15, kq = 4 * (lane >> 4);
  const float* ap[2];
  const float* bp[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = min(m0 + 16 * i + r, M - 1);
    ap[i] = A + (size_t)row * lda + kbeg + kq;
    bp[i] = W + (size_t)(n0 + 16 * i + r) * ldw + kbeg + kq;
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int nsteps = klen >> 4;
  f4 ra[PF][2], rb[PF][2];
  auto load = [&](int p, int t) {
    const int o = 16 * min(t, nsteps - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ra[p][i] = *(const f4*)(ap[i] + o);
      rb[p][i] = *(const f4*)(bp[i] + o);
    }
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) load(p, p);
  for (int t0 = 0; t0 < nsteps; t0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      if (t0 + p < nsteps) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ra[p][i][s], rb[p][j][s], acc[i][j], 0, 0, 0);
      }
      load(p, t0 + p + PF);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + 16 * i + 4 * (lane >> 4) + e;
        const int col = n0 + 16 * j + r;
        if (row >= M) continue;
        const float v = acc[i][j][e];
        if constexpr (EPI == EPI_PART) {
          C[((size_t)blockIdx.y * M + row) * ldc + col] = v;
        } else {
          const float y = bias ? v + bias[col] : v;
          C[(size_t)row * ldc + col] = y;
        }
      }
}

// out[t][n] = act(((part0 + part1) + ... + part{S-1}) + bias)  (fixed order), four
// consecutive elements per thread; all S loads are issued before the sum.
template <bool GELU, int S>
__global__ __launch_bounds__(256) void k_pf_sum(const float* __restrict__ part, int MN, int N,
                                               const float* __restrict__ bias, float* __restrict__ out) {
  const int i = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (i >= MN) return;
  f4 p[S];
#pragma unroll
  for (int s = 0; s < S; ++s) p[s] = *(const f4*)(part + (size_t)s * MN + i);
  f4 v = p[0];
#pragma unroll
  for (int s = 1; s < S; ++s) v = v + p[s];
  v = v + *(const f4*)(bias + i % N);
  if (GELU) {
    v.x = gelu_tanh(v.x);
    v.y = gelu_tanh(v.y);
    v.z = gelu_tanh(v.z);
    v.w = gelu_tanh(v.w);
  }
  *(f4*)(out + i) = v;
}

// One wave per row t: x[t] += (sum of the S parts, fixed order) + bias; then, when
// gamma is given, h[t] = LayerNorm(x[t]).
template <int S>
__global__ __launch_bounds__(64) void k_pf_resid_ln(const float* __restrict__ part, int M,
                                                    const float* __restrict__ bias, float* __restrict__ x,
                                                    const float* gamma, const float* beta, float* __restrict__ h) {
  const int t = blockIdx.x, l = lane_id();
  f4 p[3][S];
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int s = 0; s < S; ++s) p[i][s] = *(const f4*)(part + ((size_t)s * M + t) * D + 256 * i + 4 * l);
  f4 v[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    f4 a = p[i][0];
#pragma unroll
    for (int s = 1; s < S; ++s) a = a + p[i][s];
    const size_t o = (size_t)t * D + 256 * i + 4 * l;
    v[i] = *(const f4*)(x + o) + (a + *(const f4*)(bias + 256 * i + 4 * l));
  }
  store_frag<3>(x + (size_t)t * D, v);
  if (gamma) {
    layernorm_frag(v, gamma, beta);
    store_frag<3>(h + (size_t)t * D, v);
  }
}

struct Toks {
  uint32_t t[PMAX];
};

// x[t] = wte[tok_t] + wpe[t]; h[t] = LayerNorm1 of block 0 (x[t]).  One wave per row.
__global__ __launch_bounds__(64) void k_pf_embed_ln(const Weights w, const Toks tk, float* __restrict__ x,
                                                    const float* gamma, const float* beta, float* __restrict__ h) {
  const int t = blockIdx.x;
  f4 e[3], p[3];
  load_frag<3>(e, w.wte + (size_t)tk.t[t] * D);
  load_frag<3>(p, w.wpe + (size_t)t * D);
#pragma unroll
  for (int i = 0; i < 3; ++i) e[i] = e[i] + p[i];
  store_frag<3>(x + (size_t)t * D, e);
  layernorm_frag(e, gamma, beta);
  store_frag<3>(h + (size_t)t * D, e);
}

constexpr int PF_ROWS = 8;  // query rows per attention workgroup (2 per wave)

struct PfAttnSmem {
  float k[PMAX][DH + 4];
  float v[PMAX][DH];
  float q[4][DH];
  float w[4][PMAX];
};

// Causal attention of head blockIdx.x for query rows t0..t0+7 (t0 = 8*blockIdx.y)
// over the row-batch QKV buffer [n][3D].  Wave w takes rows t0+w and t0+w+4: lane j
// scores keys j and j+64, the softmax maximum and sum are wave reductions, and
// lane d sums w_j * v_j[d] over j ascending.
__global__ __launch_bounds__(256) void k_pf_attn(const float* __restrict__ qkv, int n, float* __restrict__ att) {
  __shared__ PfAttnSmem sm;
  const int h = blockIdx.x, t0 = PF_ROWS * blockIdx.y;
  const int tend = min(t0 + PF_ROWS, n);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // Stage rows 0..tend-1: 16 threads per row, each 16 keys and 16 values.  All
  // loads are issued before any store (indexes past the last row re-read it).
  {
    constexpr int U = PMAX * 16 / 256;
    f4 kk[U], vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = threadIdx.x + 256 * u;
      const int j = min(idx >> 4, tend - 1), c = (idx & 15) * 4;
      const float* row = qkv + (size_t)j * D3 + h * DH;
      kk[u] = *(const f4*)(row + D + c);
      vv[u] = *(const f4*)(row + 2 * D + c);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = threadIdx.x + 256 * u;
      const int j = idx >> 4, c = (idx & 15) * 4;
      if (j < tend) {
        *(f4*)&sm.k[j][c] = kk[u];
        *(f4*)&sm.v[j][c] = vv[u];
      }
    }
  }
  __syncthreads();
  for (int t = t0 + wave; t < tend; t += 4) {
    sm.q[wave][lane] = qkv[(size_t)t * D3 + h * DH + lane];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    float s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = lane + 64 * u;
      s[u] = -INFINITY;
      if (j <= t) {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < DH / 4; ++i) {
          const f4 kk = *(const f4*)&sm.k[j][4 * i];
          const f4 qq = *(const f4*)&sm.q[wave][4 * i];
          acc = acc + qq.x * kk.x;
          acc = acc + qq.y * kk.y;
          acc = acc + qq.z * kk.z;
          acc = acc + qq.w * kk.w;
        }
        s[u] = acc * 0.125f;
      }
    }
    const float m = wave_max(fmaxf(s[0], s[1]));
    float e[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) e[u] = lane + 64 * u <= t ? exp_spec(s[u] - m) : 0.0f;
    const float Z = wave_sum(e[0] + e[1]);
#pragma unroll
    for (int u = 0; u < 2; ++u) sm.w[wave][lane + 64 * u] = e[u] / Z;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    float o = 0.0f;
#pragma unroll 8
    for (int j = 0; j <= t; ++j) o = o + sm.w[wave][j] * sm.v[j][lane];
    att[(size_t)t * D + h * DH + lane] = o;
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_head_f32(const Weights& w, const float* x_row, float* logits, hipStream_t s);

// Split-K factors: the K range of every projection is cut into S equal runs of
// whole 16-element steps; N/32 column tiles x S workgroups per launch.
constexpr int S_QKV = 3, S_O = 8, S_FC = 2, S_PR = 8;
static_assert((size_t)S_QKV * D3 * PMAX <= PF_PART_WORDS && (size_t)S_FC * F * PMAX <= PF_PART_WORDS &&
                  (size_t)S_O * D * PMAX <= PF_PART_WORDS && (size_t)S_PR * D * PMAX <= PF_PART_WORDS,
              "partial-sum buffer");
static_assert(D % (16 * S_QKV) == 0 && D % (16 * S_O) == 0 && D % (16 * S_FC) == 0 && F % (16 * S_PR) == 0,
              "split K ranges are whole 16-element steps");

template <int EPI>
static void mm(const float* A, int lda, const float* W, int K, int M, int N, const float* bias, float* C, int ldc,
               int split, hipStream_t s) {
  const dim3 grid(N / 32, split);
  const int klen = K / split, steps = klen / 16;
  if (steps % 4 == 0)
    hipLaunchKernelGGL((k_mm<EPI, 4>), grid, dim3(256), 0, s, A, lda, W, K, M, N, bias, C, ldc, klen);
  else
    hipLaunchKernelGGL((k_mm<EPI, 2>), grid, dim3(256), 0, s, A, lda, W, K, M, N, bias, C, ldc, klen);
}

hipError_t launch_infer(const Weights& w, const Work& k, const uint32_t* toks, int n, float* logits,
                        hipStream_t s) {
  Toks tk{};
  for (int t = 0; t < n; ++t) tk.t[t] = toks[t];
  hipLaunchKernelGGL(k_pf_embed_ln, dim3(n), dim3(64), 0, s, w, tk, k.pf_x, small_p(w, 0, sp::LN1_G),
                     small_p(w, 0, sp::LN1_B), k.pf_h);
  for (int l = 0; l < L; ++l) {
    mm<EPI_PART>(k.pf_h, D, f32_mat(w, l, M_QKV), D, n, D3, nullptr, k.pf_part, D3, S_QKV, s);
    hipLaunchKernelGGL((k_pf_sum<false, S_QKV>), dim3((n * D3 / 4 + 255) / 256), dim3(256), 0, s, k.pf_part,
                       n * D3, D3, small_p(w, l, sp::B_QKV), k.pf_qkv);
    hipLaunchKernelGGL(k_pf_attn, dim3(H, (n + PF_ROWS - 1) / PF_ROWS), dim3(256), 0, s, k.pf_qkv, n, k.pf_att);
    mm<EPI_PART>(k.pf_att, D, f32_mat(w, l, M_O), D, n, D, nullptr, k.pf_part, D, S_O, s);
    hipLaunchKernelGGL(k_pf_resid_ln<S_O>, dim3(n), dim3(64), 0, s, k.pf_part, n, small_p(w, l, sp::B_O), k.pf_x,
                       small_p(w, l, sp::LN2_G), small_p(w, l, sp::LN2_B), k.pf_h);
    mm<EPI_PART>(k.pf_h, D, f32_mat(w, l, M_FC), D, n, F, nullptr, k.pf_part, F, S_FC, s);
    hipLaunchKernelGGL((k_pf_sum<true, S_FC>), dim3((n * F / 4 + 255) / 256), dim3(256), 0, s, k.pf_part, n * F,
                       F, small_p(w, l, sp::B_FC), k.pf_u);
    mm<EPI_PART>(k.pf_u, F, f32_mat(w, l, M_PR), F, n, D, nullptr, k.pf_part, D, S_PR, s);
    const bool last = l + 1 == L;
    hipLaunchKernelGGL(k_pf_resid_ln<S_PR>, dim3(n), dim3(64), 0, s, k.pf_part, n, small_p(w, l, sp::B_PR), k.pf_x,
                       last ? nullptr : small_p(w, l + 1, sp::LN1_G), last ? nullptr : small_p(w, l + 1, sp::LN1_B),
                       k.pf_h);
  }
  return launch_head_f32(w, k.pf_x + (size_t)(n - 1) * D, logits, s);
}

hipError_t launch_gemm_test(const float* A, const float* W, float* C, int M, int N, int K, hipStream_t s) {
  mm<EPI_STORE>(A, K, W, K, M, N, nullptr, C, N, 1, s);
  return hipGetLastError();
}

}  // namespace g2
