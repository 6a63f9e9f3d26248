// Full-prefix inference (LeanExe GPT-2 README, infer paragraph): 1..128 tokens run
// as row batches through the 12 blocks; only the final row reaches the tied head.
//
// The block projections are dense T x K by K x N contractions on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32 and _16x16x4_f32).  With T <= 128 rows every
// projection is short and wide: a workgroup owns all rows and 16 or 32 output
// columns, stages both operands through LDS, and the launches have 192-216
// workgroups, about one per compute unit.  FC runs over all of K in 16-column tiles
// with the bias and GELU in its epilogue.  QKV, O and the MLP projection split K;
// their partial sums are added in split order by the kernel that consumes them
// (attention for QKV, which also adds the bias; the residual-and-LayerNorm kernel
// for the other two), so results do not depend on timing.  Causal attention stages
// each head's key/value rows in LDS once per eight query rows.
#include <mutex>

#include "device.hpp"
#include "internal.hpp"

namespace g2 {

typedef float f32x16 __attribute__((ext_vector_type(16)));

enum Epi { EPI_STORE = 0, EPI_PART = 1 };

// C = A[M][K] * W[N][K]^T over the K range [z*klen, (z+1)*klen) (z = blockIdx.y) for
// the workgroup's 32 output columns n0 = 32*blockIdx.x.  Four waves; wave w computes
// rows 32w..32w+31 with v_mfma_f32_32x32x2_f32: lane l supplies A[l%32][k] and
// B[k][l%32] for k = l/32, and result register r of lane l is
// C[8(r/4) + 4(l/32) + r%4][l%32].
// K is streamed in stages of GK = 32 elements.  A stage (the GM = 128 activation rows
// and the 32 weight rows, 128 bytes each: 20 KB) is copied from memory straight into
// one of NBUF LDS buffers by 16-byte direct-to-LDS loads, NBUF-1 stages ahead of the
// one being multiplied, so no registers and no LDS store instructions carry the
// operands.  A 1 KB region of a buffer holds eight rows, chunk c of row r at slot
// c ^ ((r / 2) % 8): the LDS serves a 16-byte-per-lane read sixteen lanes at a time
// over 64 four-byte banks, and the sixteen lanes of an MFMA operand read take the
// same chunk of sixteen consecutive rows (128 bytes apart, so two rows share a
// bank offset), which this puts on distinct banks.  Each wave copies five of the
// 20 regions; it waits until its own copies of a stage have landed, and a workgroup
// barrier then makes the whole stage visible (and frees the buffer of the stage
// before, which the copies of stage t+NBUF-1 overwrite).
// Within a stage, lane half h = l/32 reads chunk 2q + h (q < 4) of its operand rows,
// and sub-step s of that chunk feeds element 8q + 4h + s, so the 32 elements are
// consumed once each; even and odd q accumulate into separate registers, added at the
// end.  Rows at or past M read row M-1 and store nothing.  Past the last stage the
// copies re-read it into a buffer no later stage uses, so every wave issues the same
// copies and the wait counts stay exact.
// EPI_STORE: C = acc + bias (bias may be null); EPI_PART: part[z][row][col] = acc.
constexpr int GK = 32;
constexpr int GM = 128;
#ifndef PF_MM_NBUF
#define PF_MM_NBUF 4
#endif
constexpr int MM_NBUF = PF_MM_NBUF;                     // stage buffers in LDS
constexpr int MM_ROWS = GM + 32;                        // staged rows per stage
constexpr int MM_BUF = MM_ROWS * GK * 4;                // bytes of one stage buffer
constexpr int MM_PERW = MM_ROWS / 8 / 4;                // 1 KB regions copied per wave per stage
constexpr int MM_LDS = MM_NBUF * MM_BUF;
static_assert(MM_PERW * 4 * 8 == MM_ROWS, "whole regions per wave");
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm(const float* __restrict__ A, int lda, const float* __restrict__ W,
                                              int ldw, int M, const float* __restrict__ bias, float* __restrict__ C,
                                              int ldc, int klen) {
  extern __shared__ __align__(16) char lds[];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n0 = 32 * blockIdx.x, kbeg = blockIdx.y * klen;
  const int nsteps = klen / GK;
  const float* src[MM_PERW];
#pragma unroll
  for (int i = 0; i < MM_PERW; ++i) {
    const int row = 8 * (wave + 4 * i) + lane / 8, c = (lane % 8) ^ ((row >> 1) & 7);
    src[i] = (row < GM ? A + (size_t)min(row, M - 1) * lda : W + (size_t)(n0 + row - GM) * ldw) + kbeg + 4 * c;
  }
  auto copy_stage = [&](int t) {
    const int o = GK * min(t, nsteps - 1);
    char* buf = lds + (t % MM_NBUF) * MM_BUF;
#pragma unroll
    for (int i = 0; i < MM_PERW; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + o),
                                       (__attribute__((address_space(3))) void*)(buf + 1024 * (wave + 4 * i)), 16, 0, 0);
  };
  const int h = lane >> 5, sw = ((lane & 31) >> 1) & 7;  // (row / 2) % 8 of the lane's A and B rows
  const int aoff = (32 * wave + (lane & 31)) * (GK * 4), boff = (GM + (lane & 31)) * (GK * 4);
  f32x16 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
#pragma unroll
  for (int p = 0; p < MM_NBUF - 1; ++p) copy_stage(p);
  // s_waitcnt with vmcnt = (NBUF-2) copies-per-stage still in flight, expcnt and
  // lgkmcnt left at their maxima
  constexpr int WAITN = (MM_NBUF - 2) * MM_PERW;
  constexpr int WAIT_STAGE = (WAITN & 15) | ((WAITN >> 4) << 14) | 0x70 | 0xF00;
  for (int t = 0; t < nsteps; ++t) {
    __builtin_amdgcn_s_waitcnt(WAIT_STAGE);  // this wave's copies of stage t have landed
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();            // and every wave's; stage t-1's buffer is free
    asm volatile("" ::: "memory");
    const char* b = lds + (t % MM_NBUF) * MM_BUF;
    f4 fa[4], fb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int slot = 16 * ((2 * q + h) ^ sw);
      fa[q] = *(const f4*)(b + aoff + slot);
      fb[q] = *(const f4*)(b + boff + slot);
    }
    copy_stage(t + MM_NBUF - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc[q & 1] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[q][s], fb[q][s], acc[q & 1], 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // no copy in flight when the workgroup ends
  const int col = n0 + (lane & 31);
  const float bv = (EPI == EPI_STORE && bias) ? bias[col] : 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 32 * wave + 8 * (r >> 2) + 4 * h + (r & 3);
    if (row >= M) continue;
    const float v = acc[0][r] + acc[1][r];
    if constexpr (EPI == EPI_PART)
      C[((size_t)blockIdx.y * M + row) * ldc + col] = v;
    else
      C[(size_t)row * ldc + col] = v + bv;
  }
}

// Narrow full-K variant for the MLP's first projection (FC): a workgroup owns all
// 128 rows and 16 output columns over the whole of K, so no split partial sums
// and no reduction launch are needed; the epilogue adds the bias (and applies
// GELU).  Eight waves, wave w computing rows 16w..16w+15 with
// v_mfma_f32_16x16x4_f32: lane l supplies A[l%16][k] and B[k][l%16] with its
// K-group kg = l/16, and result register r of lane l is C[4(l/16) + r][l%16].
// K is staged KS elements at a time (CH = KS/4 chunks of 16 bytes per row, chunk c
// of row r at slot c ^ ((r / 2) % 8), as in k_gemm); group kg reads chunks kg*CH/4 .. (kg+1)*CH/4 - 1 of
// its operand rows, and product s (< KS/4) of a stage feeds element kg*KS/4 + s,
// so a stage's elements are consumed once each.  Loads are held in registers PF
// stages ahead; a pass reads the next stage's fragments before multiplying the
// current one's, then stores stage t+2 into the buffer stage t occupied.  The
// stage's 16 weight rows are read by the first 16*CH threads (the others re-read
// one of those chunks and do not store it, so every thread issues the same loads).
constexpr int G16_NTH = 512;
template <int KS>
struct G16 {
  static constexpr int CH = KS / 4, ROWS = GM + 16, RB = KS * 4, BUF = ROWS * RB;
  static constexpr int UA = GM * CH / G16_NTH, U = UA + 1, NB = 16 * CH;
  static_assert(UA * G16_NTH == GM * CH && NB <= G16_NTH, "whole chunks per thread");
};
template <int KS, bool GELU, int PF>
__global__ __launch_bounds__(G16_NTH) void k_gemm16(const float* __restrict__ A, int lda, const float* __restrict__ W,
                                                   int ldw, int M, int K, const float* __restrict__ bias,
                                                   float* __restrict__ C, int ldc) {
  using G = G16<KS>;
  static_assert(PF % 2 == 0, "the LDS buffer of a stage follows from the unrolled pass");
  extern __shared__ __align__(16) char lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = 16 * blockIdx.x;
  const int nsteps = K / KS;
  const float* src[G::U];
  int dst[G::U];
#pragma unroll
  for (int u = 0; u < G::U; ++u) {
    const int idx = u < G::UA ? (int)threadIdx.x + G16_NTH * u : GM * G::CH + ((int)threadIdx.x % G::NB);
    const int rr = idx / G::CH, c = idx % G::CH;
    src[u] = (u < G::UA ? A + (size_t)min(rr, M - 1) * lda : W + (size_t)(n0 + rr - GM) * ldw) + 4 * c;
    dst[u] = rr * G::RB + 16 * (c ^ ((rr >> 1) & 7));
  }
  const bool bstore = (int)threadIdx.x < G::NB;
  f4 pre[PF][G::U];
  auto gload = [&](int slot, int t) {
    const int o = KS * min(t, nsteps - 1);
#pragma unroll
    for (int u = 0; u < G::U; ++u)
      pre[slot][u] = u < G::UA ? *(const f4*)(src[u] + o) : __builtin_nontemporal_load((const f4*)(src[u] + o));
  };
  auto lstore = [&](int slot, int buf) {
#pragma unroll
    for (int u = 0; u < G::U; ++u)
      if (u < G::UA || bstore) *(f4*)(lds + buf * G::BUF + dst[u]) = pre[slot][u];
  };
  constexpr int FR = G::CH / 4;  // chunks per K-group per stage
  const int kg = lane >> 4, sw = ((lane & 15) >> 1) & 7;  // (row / 2) % 8 of the lane's A and B rows
  const int aoff = (16 * wave + (lane & 15)) * G::RB, boff = (GM + (lane & 15)) * G::RB;
  auto lread = [&](f4 (&fa)[FR], f4 (&fb)[FR], int buf) {
    const char* b = lds + buf * G::BUF;
#pragma unroll
    for (int h = 0; h < FR; ++h) {
      const int slot = 16 * ((FR * kg + h) ^ sw);
      fa[h] = *(const f4*)(b + aoff + slot);
      fb[h] = *(const f4*)(b + boff + slot);
    }
  };
  f4 acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
  f4 fa[2][FR], fb[2][FR];
  // stages 0 and 1 into the two LDS buffers, stages 2..PF+1 in flight
#pragma unroll
  for (int p = 0; p < PF; ++p) gload(p, p);
  lstore(0, 0);
  gload(0, PF);
  lstore(1, 1);
  gload(1, PF + 1);
  __syncthreads();
  lread(fa[0], fb[0], 0);
  __syncthreads();  // pass 0 overwrites buffer 0
  for (int t0 = 0; t0 < nsteps; t0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int cur = p & 1;
      lread(fa[cur ^ 1], fb[cur ^ 1], cur ^ 1);
      if (t0 + p < nsteps) {
#pragma unroll
        for (int h = 0; h < FR; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[e & 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[cur][h][e], fb[cur][h][e], acc[e & 1], 0, 0, 0);
      }
      const int sl = (p + 2) % PF;
      lstore(sl, cur);
      gload(sl, t0 + p + 2 + PF);
      __syncthreads();
    }
  }
  const int col = n0 + (lane & 15);
  const float bv = bias[col];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 16 * wave + 4 * kg + r;
    if (row >= M) continue;
    float y = (acc[0][r] + acc[1][r]) + bv;
    if (GELU) y = gelu_f32(y);
    C[(size_t)row * ldc + col] = y;
  }
}

// Stage depth of the full-K kernel (K elements per LDS stage) and its launch.
constexpr int G16_KS = 32;
#ifndef PF_G16_PF
#define PF_G16_PF 2
#endif
constexpr int G16_PF = PF_G16_PF;  // stages held in registers ahead of the LDS pair
template <bool GELU>
static hipError_t gemm16(const float* A, int lda, const float* W, int M, int N, int K, const float* bias, float* C,
                         int ldc, hipStream_t s) {
  constexpr size_t lds = 2 * (size_t)G16<G16_KS>::BUF;
  hipLaunchKernelGGL((k_gemm16<G16_KS, GELU, G16_PF>), dim3(N / 16), dim3(G16_NTH), lds, s, A, lda, W, K, M, K, bias, C, ldc);
  return hipGetLastError();
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

constexpr int PF_ROWS = 8;  // query rows per attention workgroup (one per wave)
constexpr int PF_ATT_THREADS = 64 * PF_ROWS;

struct PfAttnSmem {
  float k[PMAX][DH + 4];  // padded rows: lane j reading row j hits distinct banks
  float v[PMAX][DH];
  float q[PF_ROWS][DH];
  float w[PF_ROWS][PMAX + 4];  // padded: the eight rows' reads of one column hit distinct banks
  float part[PF_ROWS][PF_ROWS][DH];  // per-wave partial weighted sums [wave][row][d]
};

// Causal attention of head blockIdx.x for query rows t0..t0+7 (t0 = 8*blockIdx.y).
// The QKV projection arrives as SP split-K partial sums part[z][t][3D] (z < SP); a
// staged value is ((part[0] + part[1]) + ...) + bias.  The key/value rows 0..t0+7
// and the eight query rows are staged in LDS once; kv (or null) also receives the
// keys and values of rows t0..t0+7, at kv[t * 12 * 1536 + col - 768] for projection
// column col >= 768, the cachedStep layout of position t for the layer kv points at
// (the prefill's handoff to the cached step).  Wave w then takes row t = t0 + w: lane j
// scores keys j and j+64 (four interleaved partial dot products), and the softmax
// maximum and sum are wave reductions.  The weighted sums are split over the keys:
// wave w sums keys 16w..16w+15 for all eight rows and 64 outputs (lane l: row l/8,
// outputs 8(l%8)..+7), and the eight partial sums are added in wave order.
template <int SP>
__global__ __launch_bounds__(PF_ATT_THREADS) void k_pf_attn(const float* __restrict__ part, const float* __restrict__ bias,
                                                            int n, float* __restrict__ att, float* __restrict__ kv) {
  __shared__ __align__(16) PfAttnSmem sm;
  const int h = blockIdx.x, t0 = PF_ROWS * blockIdx.y;
  const int tend = min(t0 + PF_ROWS, n);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t pstride = (size_t)n * D3;
  auto sum_parts = [&](const float* p) {
    f4 v = *(const f4*)p;
#pragma unroll
    for (int z = 1; z < SP; ++z) v = v + *(const f4*)(p + z * pstride);
    return v;
  };
  // Stage rows 0..tend-1: 16 threads per row, each four keys and four values, and the
  // query rows (indexes past the last row re-read it; all loads before any store).
  {
    constexpr int U = PMAX * 16 / PF_ATT_THREADS;
    f4 kk[U], vv[U], qq;
    const int qr = threadIdx.x >> 4, qc = (threadIdx.x & 15) * 4;  // 128 threads: 8 rows x 16 float4
    const f4 bk = *(const f4*)(bias + D + h * DH + (threadIdx.x & 15) * 4);
    const f4 bvv = *(const f4*)(bias + 2 * D + h * DH + (threadIdx.x & 15) * 4);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = threadIdx.x + PF_ATT_THREADS * u;
      const int j = min(idx >> 4, tend - 1), c = (idx & 15) * 4;
      const float* row = part + (size_t)j * D3 + h * DH + c;
      kk[u] = sum_parts(row + D) + bk;
      vv[u] = sum_parts(row + 2 * D) + bvv;
    }
    if (threadIdx.x < PF_ROWS * 16)
      qq = sum_parts(part + (size_t)min(t0 + qr, tend - 1) * D3 + h * DH + qc) + *(const f4*)(bias + h * DH + qc);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = threadIdx.x + PF_ATT_THREADS * u;
      const int j = idx >> 4, c = (idx & 15) * 4;
      if (j < tend) {
        *(f4*)&sm.k[j][c] = kk[u];
        *(f4*)&sm.v[j][c] = vv[u];
        if (kv && j >= t0) {
          *(f4*)(kv + (size_t)j * CACHE_POS + h * DH + c) = kk[u];
          *(f4*)(kv + (size_t)j * CACHE_POS + D + h * DH + c) = vv[u];
        }
      }
    }
    if (threadIdx.x < PF_ROWS * 16) *(f4*)&sm.q[qr][qc] = qq;
  }
  __syncthreads();
  const int t = t0 + wave;
  if (t < tend) {
    float s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = lane + 64 * u;
      s[u] = -INFINITY;
      if (j <= t) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < DH / 4; ++i) {
          const f4 kv = *(const f4*)&sm.k[j][4 * i];
          const f4 qv = *(const f4*)&sm.q[wave][4 * i];
          acc[i & 3] = fmaf(qv.x, kv.x, acc[i & 3]);
          acc[i & 3] = fmaf(qv.y, kv.y, acc[i & 3]);
          acc[i & 3] = fmaf(qv.z, kv.z, acc[i & 3]);
          acc[i & 3] = fmaf(qv.w, kv.w, acc[i & 3]);
        }
        s[u] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * 0.125f;
      }
    }
    const float m = wave_max(fmaxf(s[0], s[1]));
    float e[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) e[u] = lane + 64 * u <= t ? exp_f32(s[u] - m) : 0.0f;
    const float Z = wave_sum(e[0] + e[1]);
    const float rz = __builtin_amdgcn_rcpf(Z);  // Z >= 1 (the maximum's term is 1)
#pragma unroll
    for (int u = 0; u < 2; ++u) sm.w[wave][lane + 64 * u] = e[u] * rz;
  } else {
#pragma unroll
    for (int u = 0; u < 2; ++u) sm.w[wave][lane + 64 * u] = 0.0f;
  }
  __syncthreads();
  // weighted sums over keys 16w..16w+15 (weights past a row's own position are 0;
  // keys past tend-1 are not staged and contribute nothing)
  {
    const int r = lane >> 3, d0 = 8 * (lane & 7), j0 = 16 * wave;
    f4 o0 = {0.0f, 0.0f, 0.0f, 0.0f}, o1 = {0.0f, 0.0f, 0.0f, 0.0f};
    if (j0 < tend) {
#pragma unroll
      for (int jj = 0; jj < 16; jj += 4) {
        const f4 wv = *(const f4*)&sm.w[r][j0 + jj];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = min(j0 + jj + i, tend - 1);  // a weight-0 key past tend-1 reads the last staged row
          const float wj = i == 0 ? wv.x : i == 1 ? wv.y : i == 2 ? wv.z : wv.w;
          const f4 v0 = *(const f4*)&sm.v[j][d0], v1 = *(const f4*)&sm.v[j][d0 + 4];
          o0.x = fmaf(wj, v0.x, o0.x);
          o0.y = fmaf(wj, v0.y, o0.y);
          o0.z = fmaf(wj, v0.z, o0.z);
          o0.w = fmaf(wj, v0.w, o0.w);
          o1.x = fmaf(wj, v1.x, o1.x);
          o1.y = fmaf(wj, v1.y, o1.y);
          o1.z = fmaf(wj, v1.z, o1.z);
          o1.w = fmaf(wj, v1.w, o1.w);
        }
      }
    }
    *(f4*)&sm.part[wave][r][d0] = o0;
    *(f4*)&sm.part[wave][r][d0 + 4] = o1;
  }
  __syncthreads();
  {
    const int r = threadIdx.x >> 6, d = threadIdx.x & 63;  // one output per thread
    float acc = sm.part[0][r][d];
#pragma unroll
    for (int w2 = 1; w2 < PF_ROWS; ++w2) acc = acc + sm.part[w2][r][d];
    if (t0 + r < tend) att[(size_t)(t0 + r) * D + h * DH + d] = acc;
  }
}

hipError_t launch_head_f32(const Weights& w, const float* x_row, float* logits, hipStream_t s);

// Split-K factors: the K range of a projection is cut into S equal runs of whole
// GK-element stages; N/32 column tiles x S workgroups per launch (QKV: 216, O and
// MLP projection: 192).  The partial sums are added in split order by the kernel
// that consumes them (attention for QKV, the residual-and-LayerNorm kernel for O
// and the MLP projection).
// QKV's split can be set at build time (-DPF_S_QKV=2 or 4 fit the partial-sum
// buffer and divide K = 768 into whole stages); 3 measured fastest.
#ifndef PF_S_QKV
#define PF_S_QKV 3
#endif
#ifndef PF_S_O
#define PF_S_O 8
#endif
#ifndef PF_S_PR
#define PF_S_PR 8
#endif
constexpr int S_QKV = PF_S_QKV, S_O = PF_S_O, S_PR = PF_S_PR;
static_assert((size_t)S_QKV * D3 * PMAX <= PF_PART_WORDS && (size_t)S_O * D * PMAX <= PF_PART_WORDS &&
                  (size_t)S_PR * D * PMAX <= PF_PART_WORDS,
              "partial-sum buffer");
static_assert(D % (GK * S_QKV) == 0 && D % (GK * S_O) == 0 && F % (GK * S_PR) == 0, "split K ranges are whole stages");
static_assert(D3 % 32 == 0 && D % 32 == 0, "k_gemm column tiles");
static_assert(F % 16 == 0 && D % G16_KS == 0, "k_gemm16 tiles");

// N must be a multiple of 32, K of GK * split, 1 <= M <= GM.
template <int EPI>
static hipError_t mm(const float* A, int lda, const float* W, int K, int M, int N, const float* bias, float* C, int ldc,
                     int split, hipStream_t s) {
  hipLaunchKernelGGL((k_gemm<EPI>), dim3(N / 32, split), dim3(256), MM_LDS, s, A, lda, W, K, M, bias, C, ldc, K / split);
  return hipGetLastError();
}

// The GEMM kernels' LDS limits, set once per process (thread-safe) before their first launch.
static hipError_t prefill_attrs() {
  static std::once_flag once;
  static hipError_t err = hipSuccess;
  std::call_once(once, [] {
    const void* fs[] = {(const void*)k_gemm<EPI_PART>, (const void*)k_gemm<EPI_STORE>};
    for (const void* f : fs)
      if (err == hipSuccess) err = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, MM_LDS);
    const void* gs[] = {(const void*)k_gemm16<G16_KS, true, G16_PF>, (const void*)k_gemm16<G16_KS, false, G16_PF>};
    for (const void* f : gs)
      if (err == hipSuccess)
        err = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 2 * (int)G16<G16_KS>::BUF);
  });
  return err;
}

hipError_t launch_infer(const Weights& w, const Work& k, const uint32_t* toks, int n, float* logits,
                        hipStream_t s, float* cache) {
  Toks tk{};
  hipError_t e;
  if ((e = prefill_attrs())) return e;
  for (int t = 0; t < n; ++t) tk.t[t] = toks[t];
  hipLaunchKernelGGL(k_pf_embed_ln, dim3(n), dim3(64), 0, s, w, tk, k.pf_x, small_p(w, 0, sp::LN1_G),
                     small_p(w, 0, sp::LN1_B), k.pf_h);
  for (int l = 0; l < L; ++l) {
    if ((e = mm<EPI_PART>(k.pf_h, D, f32_mat(w, l, M_QKV), D, n, D3, nullptr, k.pf_part, D3, S_QKV, s))) return e;
    hipLaunchKernelGGL(k_pf_attn<S_QKV>, dim3(H, (n + PF_ROWS - 1) / PF_ROWS), dim3(PF_ATT_THREADS), 0, s, k.pf_part,
                       small_p(w, l, sp::B_QKV), n, k.pf_att, cache ? cache + (size_t)l * KV_ROW : nullptr);
    if ((e = mm<EPI_PART>(k.pf_att, D, f32_mat(w, l, M_O), D, n, D, nullptr, k.pf_part, D, S_O, s))) return e;
    hipLaunchKernelGGL(k_pf_resid_ln<S_O>, dim3(n), dim3(64), 0, s, k.pf_part, n, small_p(w, l, sp::B_O), k.pf_x,
                       small_p(w, l, sp::LN2_G), small_p(w, l, sp::LN2_B), k.pf_h);
    if ((e = gemm16<true>(k.pf_h, D, f32_mat(w, l, M_FC), n, F, D, small_p(w, l, sp::B_FC), k.pf_u, F, s))) return e;
    if ((e = mm<EPI_PART>(k.pf_u, F, f32_mat(w, l, M_PR), F, n, D, nullptr, k.pf_part, D, S_PR, s))) return e;
    const bool last = l + 1 == L;
    hipLaunchKernelGGL(k_pf_resid_ln<S_PR>, dim3(n), dim3(64), 0, s, k.pf_part, n, small_p(w, l, sp::B_PR), k.pf_x,
                       last ? nullptr : small_p(w, l + 1, sp::LN1_G), last ? nullptr : small_p(w, l + 1, sp::LN1_B),
                       k.pf_h);
  }
  return launch_head_f32(w, k.pf_x + (size_t)(n - 1) * D, logits, s);
}

hipError_t launch_gemm16_test(const float* A, const float* W, const float* bias, float* C, int M, int N, int K,
                              bool gelu, hipStream_t s) {
  if (K % G16_KS) return hipErrorInvalidValue;
  if (const hipError_t e = prefill_attrs()) return e;
  return gelu ? gemm16<true>(A, K, W, M, N, K, bias, C, N, s) : gemm16<false>(A, K, W, M, N, K, bias, C, N, s);
}

hipError_t launch_gemm_test(const float* A, const float* W, float* C, int M, int N, int K, hipStream_t s) {
  if (const hipError_t e = prefill_attrs()) return e;
  return mm<EPI_STORE>(A, K, W, K, M, N, nullptr, C, N, 1, s);
}

}  // namespace g2
