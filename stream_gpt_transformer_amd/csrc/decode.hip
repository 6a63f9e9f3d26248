// Decode-step kernels: one token per session through the 12 blocks and the tied
// head (LeanExe GPT-2 README, cachedStep paragraph), binary32 and int8 group-64
// (marXiv 2609.00018 abstract).
//
// Each phase of a block is one kernel here.  The projections stream weight rows
// with 1 KB coalesced wave loads (lane fragments, device.hpp), keep them in
// registers and apply them to every session of the launch, so a batch of B
// sessions reads each weight once and every output keeps the batch-1 arithmetic.
#include "device.hpp"
#include "internal.hpp"

namespace g2 {

enum Mode { MODE_QKV = M_QKV, MODE_O = M_O, MODE_FC = M_FC, MODE_PR = M_PR, MODE_HEAD = M_HEAD };

struct ProjArgs {
  Weights w;
  Work k;
  Sessions ss;
  float* caches;        // session b's cache starts at caches + b*cache_stride
  size_t cache_stride;  // words
  float* logits;        // [B][V]
  char* capture;        // int8 path capture buffer or null
  const uint32_t* tokp; // session 0's token in device memory, or null
  int layer;
  int qx, qw;           // int8 input / weight scale groups in units of 64 (0 = the whole row)
  int sb;               // k_proj: sessions per workgroup (blockIdx.y takes sessions sb*y ..)
  int preln;            // k_proj: LayerNorm inputs already normalised in k.att (k_bln)
};

template <class T>
__device__ __forceinline__ T nt_load(const T* p) {
  return __builtin_nontemporal_load(p);
}

// x += wte[tok] + wpe[pos]: one block of 192 threads per session (the fp32 token
// table for every weight format).
__global__ __launch_bounds__(192) void k_embed(const Weights w, const Sessions ss, float* x, const uint32_t* tokp) {
  const int b = blockIdx.x, t = threadIdx.x;
  const uint32_t tok = b == 0 && tokp ? min(*tokp, (uint32_t)V - 1) : ss.tok[b];
  const f4 e = *(const f4*)(w.wte + (size_t)tok * D + 4 * t);
  const f4 p = *(const f4*)(w.wpe + (size_t)ss.pos[b] * D + 4 * t);
  *(f4*)(x + (size_t)b * D + 4 * t) = e + p;
}

template <int MODE>
__device__ __forceinline__ constexpr int mode_rows() {
  return MODE == MODE_QKV ? D3 : MODE == MODE_FC ? F : MODE == MODE_HEAD ? V : D;
}
template <int MODE>
__device__ __forceinline__ constexpr bool mode_ln() {
  return MODE == MODE_QKV || MODE == MODE_FC || MODE == MODE_HEAD;
}

// Raw input vector of session b: the residual x (QKV, FC, HEAD take its
// LayerNorm), the attention output (O) or the GELU output (PR).
template <int MODE>
__device__ __forceinline__ const float* proj_src(const ProjArgs& a, int b) {
  return MODE == MODE_O ? a.k.att + (size_t)b * D : MODE == MODE_PR ? a.k.g + (size_t)b * F : a.k.x + (size_t)b * D;
}
template <int MODE>
__device__ __forceinline__ const float* ln_gamma(const ProjArgs& a) {
  return MODE == MODE_QKV ? small_p(a.w, a.layer, sp::LN1_G)
         : MODE == MODE_FC ? small_p(a.w, a.layer, sp::LN2_G) : a.w.small + sp::LNF_G;
}
template <int MODE>
__device__ __forceinline__ const float* ln_beta(const ProjArgs& a) {
  return MODE == MODE_QKV ? small_p(a.w, a.layer, sp::LN1_B)
         : MODE == MODE_FC ? small_p(a.w, a.layer, sp::LN2_B) : a.w.small + sp::LNF_B;
}

// fp32-path projection input of session b as a lane fragment: LN1(x), attention
// output, LN2(x), GELU output, LN_f(x) for QKV, O, FC, PR, HEAD.
template <int MODE, int NI>
__device__ __forceinline__ void proj_input(const ProjArgs& a, int b, f4 (&x)[NI]) {
  load_frag<NI>(x, proj_src<MODE>(a, b));
  if constexpr (mode_ln<MODE>()) layernorm_frag(*reinterpret_cast<f4(*)[3]>(&x), ln_gamma<MODE>(a), ln_beta<MODE>(a));
}

// Epilogue of output r of session b; y is the projection value including bias.  Q8:
// the int8 path's GELU (gelu_tanh) instead of the binary32 one (gelu_f32).
template <int MODE, bool Q8 = false>
__device__ __forceinline__ void proj_store(const ProjArgs& a, int b, int r, float y) {
  if constexpr (MODE == MODE_QKV) {
    a.k.qkv[(size_t)b * D3 + r] = y;
    if (r >= D) {
      float* cache = a.caches + (size_t)b * a.cache_stride;
      cache[((size_t)a.ss.pos[b] * L + a.layer) * KV_ROW + (r - D)] = y;
    }
  } else if constexpr (MODE == MODE_O || MODE == MODE_PR) {
    float* x = a.k.x + (size_t)b * D + r;
    *x = *x + y;
  } else if constexpr (MODE == MODE_FC) {
    a.k.g[(size_t)b * F + r] = Q8 ? gelu_tanh(y) : gelu_f32(y);
  } else {
    a.logits[(size_t)b * V + r] = y;
  }
}

template <int MODE>
__device__ __forceinline__ float proj_bias(const ProjArgs& a, int r) {
  if constexpr (MODE == MODE_QKV) return small_p(a.w, a.layer, sp::B_QKV)[r];
  else if constexpr (MODE == MODE_O) return small_p(a.w, a.layer, sp::B_O)[r];
  else if constexpr (MODE == MODE_FC) return small_p(a.w, a.layer, sp::B_FC)[r];
  else if constexpr (MODE == MODE_PR) return small_p(a.w, a.layer, sp::B_PR)[r];
  else return 0.0f;
}

// One fp32 projection output without bias: the output projection sums its 12 head
// groups and the MLP projection its 8 slices in fixed order (o_row, pr_row); the
// others are one 64-lane dot (dot_frag).
template <int MODE, int NI>
__device__ __forceinline__ float proj_dot(const f4 (&w)[NI], const f4 (&x)[NI]) {
  if constexpr (MODE == MODE_O) return o_row(w, x);
  else if constexpr (MODE == MODE_PR) return pr_row(w, x);
  else return dot_frag<NI>(w, x);
}

// fp32 projection over B sessions.  Block = 4 waves; wave w owns RPW consecutive
// output rows, whose weights it loads once; sessions are staged BT at a time in
// LDS as (normalised) input fragments.  Output r of session b is
// proj_dot(W_r, x_b) + bias_r — the same value for any B, RPW, BT or session split
// (blockIdx.y takes sessions a.sb*y .. a.sb*y + a.sb - 1).  H16: the weights are read
// as binary16 and widened (exact) when loaded.
// A pass computes the BT*RPW outputs o = s*RPW + rr (session s, row rr) of a tile
// together: every lane forms its lane partials as proj_dot does, the cross-lane
// trees run transposed over the outputs (wave_treduce, row_treduce: the same adds
// as wave_sum and row16_sum), the output projection's head chain and the MLP
// projection's slice chains run in the lanes of row 0, and each result lands in
// one lane, where its bias, epilogue (GELU, residual add, cache copy) and store run.
template <int MODE, int RPW, int BT, bool H16>
__global__ __launch_bounds__(256) void k_proj(const ProjArgs a) {
  constexpr int NI = MODE == MODE_PR ? F / 256 : D / 256;
  constexpr int K = 256 * NI;
  constexpr int NROWS = mode_rows<MODE>();
  constexpr bool FULL = MODE != MODE_O && MODE != MODE_PR;  // one 64-lane tree per output
  constexpr int NO = BT * RPW;                               // outputs of a pass
  constexpr int GN = NO < 16 ? NO : 16;                      // outputs per transposed reduction
  constexpr int NG = NO / GN;                                // reductions per pass (lane row g holds group g)
  constexpr int SG = GN / RPW;                               // sessions per group
  static_assert(NO % GN == 0 && GN % RPW == 0 && NG <= 4 && (FULL || NG == 1), "pass shape");
  __shared__ __align__(16) float xs[BT][K];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * 4 + wave) * RPW;
  const float* W = MODE == MODE_HEAD ? a.w.wte : f32_mat(a.w, a.layer, MODE);
  const uint16_t* W16 = H16 ? f16_mat(a.w, a.layer, MODE) : nullptr;
  f4 w[RPW][NI];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int r = row0 + rr;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const size_t e = (size_t)r * K + 256 * i + 4 * lane;
      if (r >= NROWS) w[rr][i] = f4{0, 0, 0, 0};
      else if constexpr (H16) w[rr][i] = widen(nt_load((const h4*)(W16 + e)));
      else w[rr][i] = nt_load((const f4*)(W + e));
    }
  }
  // the output this lane receives: group grp (lane row), output o of the pass
  const int t = lane & 15, grp = lane >> 4;
  const int o = GN * grp + treduce_out<GN>(t);
  const bool olane = grp < NG && t < GN;
  const int os = o / RPW, orow = row0 + o % RPW;
  const float bias = olane && orow < NROWS ? proj_bias<MODE>(a, orow) : 0.0f;
  const int sb1 = min(a.ss.B, (int)(blockIdx.y + 1) * a.sb);
  for (int b0 = blockIdx.y * a.sb; b0 < sb1; b0 += BT) {
    const int nb = min(BT, sb1 - b0);
    __syncthreads();
    for (int s = wave; s < nb; s += 4) {
      f4 x[NI];
      if (mode_ln<MODE>() && a.preln) load_frag<NI>(x, a.k.att + (size_t)(b0 + s) * D);
      else proj_input<MODE, NI>(a, b0 + s, x);
      store_frag<NI>(&xs[s][0], x);
    }
    __syncthreads();
    // staged rows past nb hold stale values; their outputs are never stored
    float y = 0.0f;
    if constexpr (FULL) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        float p[GN];
#pragma unroll
        for (int sl = 0; sl < SG; ++sl) {
          f4 x[NI];
          load_frag<NI>(x, &xs[g * SG + sl][0]);
#pragma unroll
          for (int rr = 0; rr < RPW; ++rr) p[sl * RPW + rr] = dot_lane<NI>(w[rr], x);
        }
        const float r = wave_treduce<GN>(p);
        y = grp == g ? r : y;
      }
    } else {
      // group sums: fragment i, lane row q holds the 64-input group 4i + q
      float gs[NI][4];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float p[GN];
#pragma unroll
        for (int sl = 0; sl < SG; ++sl) {
          const f4 xv = *(const f4*)&xs[sl][256 * i + 4 * lane];
#pragma unroll
          for (int rr = 0; rr < RPW; ++rr) p[sl * RPW + rr] = fma4(w[rr][i], xv);
        }
        const float tr = row_treduce<GN>(p);
        gs[i][0] = tr;
        gs[i][1] = row1_to_row0(tr);
        gs[i][2] = row2_to_row0(tr);
        gs[i][3] = row3_to_row0(tr);
      }
      if constexpr (MODE == MODE_O) {
        // y = 0, y = y + p_h for heads h = 0..11 (o_row)
#pragma unroll
        for (int h = 0; h < H; ++h) y = y + gs[h / 4][h % 4];
      } else {
        // p_s = q_6s + ... + q_6s+5, y = 0, y = y + p_s for s = 0..7 (pr_row)
#pragma unroll
        for (int sl = 0; sl < PR_SLICES; ++sl) {
          const int g0 = PR_SLICE_GROUPS * sl;
          float ps = gs[g0 / 4][g0 % 4];
#pragma unroll
          for (int k = 1; k < PR_SLICE_GROUPS; ++k) ps = ps + gs[(g0 + k) / 4][(g0 + k) % 4];
          y = y + ps;
        }
      }
    }
    if (olane && os < nb && orow < NROWS) proj_store<MODE>(a, b0 + os, orow, y + bias);
  }
}

// The LayerNorm input of a batched projection, once per session (proj_input's
// values), into the attention-output buffer, which is free at that point of the
// block: k_proj then reads it instead of normalising in every workgroup.
template <int MODE>
__global__ __launch_bounds__(64) void k_bln(const ProjArgs a) {
  f4 x[3];
  proj_input<MODE, 3>(a, blockIdx.x, x);
  store_frag<3>(a.k.att + (size_t)blockIdx.x * D, x);
}

// Attention of head blockIdx.x for session blockIdx.y over its positions 0..pos,
// reading every key/value row (the current one included) from the session's cache
// at (source*12 + layer)*1536 + offset.  attn_threads<SEQ>() threads: the fp32 form
// gives the same value for any multiple of 128 (the single-launch kernel runs it
// with 512); the sequential-order form takes 128.
template <bool SEQ>
constexpr int attn_threads() { return SEQ ? 128 : 512; }
template <bool SEQ>
__global__ __launch_bounds__(attn_threads<SEQ>()) void k_attn(const ProjArgs a) {
  constexpr int NT = attn_threads<SEQ>();
  __shared__ __align__(16) AttnSmem sm;
  const int h = blockIdx.x, b = blockIdx.y;
  const int npos = a.ss.pos[b] + 1;
  const float* cache = a.caches + (size_t)b * a.cache_stride;
  const int l = a.layer;
  auto kv = [&](int j) { return cache + ((size_t)j * L + l) * KV_ROW + h * DH; };
  attn_stage(sm, kv, npos, a.k.qkv + (size_t)b * D3 + h * DH, NT);
  __syncthreads();
  const float o = SEQ ? attn_compute_seq(sm, npos) : attn_compute<NT>(sm, npos);
  if (threadIdx.x < DH) a.k.att[(size_t)b * D + h * DH + threadIdx.x] = o;
}

// ---- int8 group-64 projections (batch 1) -------------------------------------
// LayerNorm inputs use the sequential-order LayerNorm, taken by the whole
// eight-wave workgroup (layernorm_seq_wg), and the attention the sequential-order
// attn_compute_seq, as the fused int8 step does.  The block quantizes its fp32 input in LDS (every block does the same work
// and gets the same codes), then each wave streams its rows' int8 codes: lane l takes
// 16 codes at byte 1024*i + 16*l, so group 16*i + l/4; v_dot4 gives a lane partial
// and two exact integer butterfly steps give the group accumulator.  The rescale
// runs in one fixed order: y = 0; y = y + ((float)acc_g * sw_g) * sx_g for
// g = 0..G-1; y = y + bias.
// Granularity variants (qx, qw other than 64-coordinate groups; marXiv 2609.00018
// abstract): an input group takes the largest magnitude of its 64-coordinate
// pieces (an exact maximum) and quant_lane's scale and code rules; the exact group
// accumulators of the gm = gcd(gx, gw) coordinates on which both scales are
// constant are integer sums of the 64-coordinate ones, and y = 0; y = y +
// ((float)acc_h * sw_h) * sx_h for h ascending; y = y + bias.
__device__ __forceinline__ int gcd_int(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}
template <int K>
__device__ __forceinline__ float q8_dot_groups(const i4 (&wc)[(K + 1023) / 1024], float swl, const int8_t* xc,
                                               const float* xsc, int qm) {
  constexpr int G = K / 64;
  const int accg = q8_group_acc<K>(wc, xc, lane_id());
  float y = 0.0f;
  for (int h = 0; h < G / qm; ++h) {
    int acc = 0;
    for (int t = 0; t < qm; ++t) acc += __builtin_amdgcn_readlane(accg, h * qm + t);
    const float sw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(swl), h * qm));
    y = y + ((float)acc * sw) * xsc[h * qm];
  }
  return y;
}

// Waves of a k_q8proj workgroup: eight (where the input is a LayerNorm output, the
// whole workgroup takes the sequential sums, layernorm_seq_wg).
__host__ __device__ constexpr int q8_waves(int) { return 8; }

template <int MODE, int RPW>
__global__ __launch_bounds__(64 * q8_waves(MODE)) void k_q8proj(const ProjArgs a) {
  constexpr int K = MODE == MODE_PR ? F : D;
  constexpr int NI = K / 256;
  constexpr int G = K / 64;
  constexpr int NCH = (K + 1023) / 1024;
  constexpr int NROWS = mode_rows<MODE>();
  constexpr int NW = q8_waves(MODE), NT = 64 * NW;
  constexpr bool LN = mode_ln<MODE>();
  static_assert(!LN || NW == 8, "layernorm_seq_wg takes 512 threads");
  __shared__ __align__(16) float xf[K];
  __shared__ __align__(16) float xn[LN ? D : 1];       // LayerNorm output
  __shared__ __align__(16) float lntmp[LN ? D : 1];
  __shared__ __align__(16) float tab[LN ? SEQ_TAB_FLOATS : 1];
  __shared__ __align__(16) int8_t xc[K];
  __shared__ float xsc[G];
  __shared__ float xm[G];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int qx = a.qx == 0 ? G : a.qx, qm = gcd_int(qx, a.qw == 0 ? G : a.qw);
  const CapLayout cl = cap_item(MODE);
  char* cap = a.capture ? a.capture + cap_offset(a.layer, MODE) : nullptr;

  // The wave's weight rows are requested first, so their latency overlaps the input's
  // load, LayerNorm and quantization; the workgroup barriers below order LDS only and
  // leave these loads in flight.  Rows past the matrix re-read its last row.
  const int8_t* codes = q8_codes(a.w, a.layer, MODE);
  const float* scales = q8_scales(a.w, a.layer, MODE);
  const int row0 = (blockIdx.x * NW + wave) * RPW;
  i4 wc[RPW][NCH];
  float swl[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) q8_load_row<K>(wc[rr], swl[rr], codes, scales, min(row0 + rr, NROWS - 1));

  if (wave == 0) {
    f4 x[NI];
    load_frag<NI>(x, proj_src<MODE>(a, 0));
    store_frag<NI>(xf, x);
  }
  lds_barrier();
  if constexpr (LN) {
    layernorm_seq_wg<2>(xf, ln_gamma<MODE>(a), ln_beta<MODE>(a), xn, lntmp, tab);
    lds_barrier();
  }
  const float* xq = LN ? xn : xf;  // the projection's input
  if (qx == 1) {
    for (int g = wave; g < G; g += NW) {
      float s;
      const int c = quant_lane(xq[g * 64 + lane], s);
      xc[g * 64 + lane] = (int8_t)c;
      if (lane == 0) xsc[g] = s;
    }
  } else {
    for (int g = wave; g < G; g += NW) {
      const float m = wave_max(fabsf(xq[g * 64 + lane]));
      if (lane == 0) xm[g] = m;
    }
    lds_barrier();
    for (int g = wave; g < G; g += NW) {
      const int g0 = g - g % qx;
      float m = 0.0f;
      for (int t = 0; t < qx; ++t) m = fmaxf(m, xm[g0 + t]);
      const float sc = m == 0.0f ? 0.0f : m / 127.0f;
      xc[g * 64 + lane] = m == 0.0f ? 0 : (int8_t)quant_code(xq[g * 64 + lane], sc);
      if (lane == 0) xsc[g] = sc;
    }
  }
  lds_barrier();
  if (cap && blockIdx.x == 0) {
    for (int i = threadIdx.x; i < K; i += NT) {
      ((float*)(cap + cl.in))[i] = xq[i];
      ((int8_t*)(cap + cl.codes))[i] = xc[i];
    }
    if (threadIdx.x < G) ((float*)(cap + cl.xs))[threadIdx.x] = xsc[threadIdx.x];
  }

#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int r = row0 + rr;
    if (r >= NROWS) break;
    int32_t* ca = cap ? (int32_t*)(cap + cl.acc) + (size_t)r * G : nullptr;
    float y = qm == 1 ? q8_dot<K>(wc[rr], swl[rr], xc, xsc, ca) : q8_dot_groups<K>(wc[rr], swl[rr], xc, xsc, qm);
    y = y + proj_bias<MODE>(a, r);
    if (cap && lane == 0) ((float*)(cap + cl.y))[r] = y;
    if (lane == 0) proj_store<MODE, true>(a, 0, r, y);
  }
}

// Stand-alone group-64 quantizer (test hook): block g quantizes x[64g .. 64g+63].
__global__ __launch_bounds__(64) void k_quantize(const float* x, int8_t* codes, float* scales) {
  const int g = blockIdx.x, lane = threadIdx.x;
  float s;
  const int c = quant_lane(x[(size_t)g * 64 + lane], s);
  codes[(size_t)g * 64 + lane] = (int8_t)c;
  if (lane == 0) scales[g] = s;
}

// Greedy choice of one generation step (the `lean` page's GPU path: the next token
// is picked on the GPU; LeanExe GPT-2 README, CLI paragraph: the host rejects
// non-finite logits).  The first maximum of the 50,257 logits: each thread loads
// indexes t, t+1024, ... at once and keeps the first strictly larger value, and
// pairs are combined by (larger value, then smaller index).  Any non-finite logit rejects the
// step: status = step + 1 (the first such step), its token and every later one is
// 50,257 (no token), and the fed token is 0.  Step 0 also resets the status.
__global__ __launch_bounds__(1024) void k_argmax(const float* __restrict__ logits, uint32_t* next,
                                                 uint32_t* tokens_out, int32_t* status, int step) {
  __shared__ float sv[16];
  __shared__ int si[16], sbad[16];
  constexpr int PER = (V + 1023) / 1024;
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {  // every load in flight before the first compare
    const int i = threadIdx.x + 1024 * j;
    v[j] = i < V ? logits[i] : -INFINITY;
  }
  float bv = -INFINITY;
  int bi = V, bad = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x + 1024 * j;
    bad |= i < V && !__builtin_isfinite(v[j]);
    if (v[j] > bv) {
      bv = v[j];
      bi = i;
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  bad = __any(bad) ? 1 : 0;
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
    sbad[wave] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w2 = 1; w2 < 16; ++w2) {
      if (sv[w2] > bv || (sv[w2] == bv && si[w2] < bi)) {
        bv = sv[w2];
        bi = si[w2];
      }
      bad |= sbad[w2];
    }
    const int before = step == 0 ? 0 : *status;
    uint32_t tok = (uint32_t)bi;
    if (before != 0 || bad || bi >= V) tok = (uint32_t)V;
    if (before == 0) *status = bad || bi >= V ? step + 1 : 0;
    tokens_out[step] = tok;
    *next = tok < (uint32_t)V ? tok : 0u;
  }
}

// The int8 path's LayerNorm by a 512-thread workgroup per row (test hook).
__global__ __launch_bounds__(512) void k_layernorm_seq(const float* x, const float* gamma, const float* beta,
                                                       float* y) {
  __shared__ __align__(16) float xs[D];
  __shared__ __align__(16) float ys[D];
  __shared__ __align__(16) float tmp[D];
  __shared__ __align__(16) float g[D];
  __shared__ __align__(16) float b[D];
  __shared__ __align__(16) float tab[SEQ_TAB_FLOATS];
  const size_t o = (size_t)blockIdx.x * D;
  for (int i = threadIdx.x; i < D; i += 512) {
    xs[i] = x[o + i];
    g[i] = gamma[i];
    b[i] = beta[i];
  }
  __syncthreads();
  layernorm_seq_wg<2>(xs, g, b, ys, tmp, tab);
  __syncthreads();
  for (int i = threadIdx.x; i < D; i += 512) y[o + i] = ys[i];
}

// The specified exponential (kind 0) or tanh (kind 1) of the binary32 value whose
// bit pattern is first + i (test hook).
__global__ __launch_bounds__(256) void k_special_bits(int kind, uint32_t first, long long n, float* y) {
  const long long i = blockIdx.x * 256ll + threadIdx.x;
  if (i >= n) return;
  const float x = __uint_as_float(first + (uint32_t)i);
  y[i] = kind == 0 ? exp_spec(x) : tanh_spec(x);
}

// ---- launchers ---------------------------------------------------------------

// Batched step (B > 1) launch shape: rows per wave (the 768-input projections; the
// MLP projection's 3,072-input rows take BATCH_RPW_PR), sessions staged per pass for
// the 768- and 3,072-input projections, sessions per workgroup (grid.y = B /
// BATCH_SB).  Four rows a wave reuse each staged input fragment for four outputs
// (0.877 -> 0.863 ms a step against two rows and eight sessions a pass).
#ifndef BATCH_RPW
#define BATCH_RPW 4
#endif
#ifndef BATCH_RPW_PR
#define BATCH_RPW_PR 2
#endif
#ifndef BATCH_BT768
#define BATCH_BT768 4
#endif
#ifndef BATCH_BT3072
#define BATCH_BT3072 4
#endif
#ifndef BATCH_SB
#define BATCH_SB 8
#endif
// 1: the LayerNorm inputs are normalised once per session (k_bln) before the
// projection; 0: every workgroup normalises the sessions it stages
#ifndef BATCH_PRELN
#define BATCH_PRELN 1
#endif
// the head (50,257 rows): more rows and sessions per workgroup, fewer input re-reads
#ifndef BATCH_HEAD_RPW
#define BATCH_HEAD_RPW 4
#endif
#ifndef BATCH_HEAD_SB
#define BATCH_HEAD_SB 64
#endif
#ifndef BATCH_HEAD_BT  // sessions staged per pass: 24 KB of LDS, so more workgroups fit a CU
#define BATCH_HEAD_BT 8
#endif

template <int MODE, int RPW, int BT, bool H16>
static void launch_proj(const ProjArgs& a, hipStream_t s) {
  const int rows = MODE == MODE_QKV ? D3 : MODE == MODE_FC ? F : MODE == MODE_HEAD ? V : D;
  const int nblk = (rows + 4 * RPW - 1) / (4 * RPW);
  hipLaunchKernelGGL((k_proj<MODE, RPW, BT, H16>), dim3(nblk, (a.ss.B + a.sb - 1) / a.sb), dim3(256), 0, s, a);
}

// With a.preln (batched step), the LayerNorm inputs are normalised once per session
// first (k_bln) and the projections read them.
template <int MODE, int RPW, int BT, bool H16>
static void launch_proj_ln(const ProjArgs& a, hipStream_t s) {
  if (a.preln) hipLaunchKernelGGL(k_bln<MODE>, dim3(a.ss.B), dim3(64), 0, s, a);
  launch_proj<MODE, RPW, BT, H16>(a, s);
}
template <int RPW, int BT768, int BT3072, bool H16, int RPW_PR = RPW>
static void launch_layers(ProjArgs& a, hipStream_t s) {
  const int B = a.ss.B;
  hipLaunchKernelGGL(k_embed, dim3(B), dim3(192), 0, s, a.w, a.ss, a.k.x, a.tokp);
  for (int l = 0; l < L; ++l) {
    a.layer = l;
    launch_proj_ln<MODE_QKV, RPW, BT768, H16>(a, s);
    hipLaunchKernelGGL(k_attn<false>, dim3(H, B), dim3(attn_threads<false>()), 0, s, a);
    launch_proj<MODE_O, RPW, BT768, H16>(a, s);
    launch_proj_ln<MODE_FC, RPW, BT768, H16>(a, s);
    launch_proj<MODE_PR, RPW_PR, BT3072, H16>(a, s);
  }
  if (B > 1) {
    ProjArgs ah = a;
    ah.sb = BATCH_HEAD_SB;
    ah.preln = 1;
    launch_proj_ln<MODE_HEAD, BATCH_HEAD_RPW, BATCH_HEAD_BT, H16>(ah, s);
  } else {
    launch_proj_ln<MODE_HEAD, RPW, BT768, H16>(a, s);
  }
}

hipError_t launch_step_f32(const Weights& w, const Work& k, const Sessions& ss, float* caches,
                           size_t cache_stride, float* logits, hipStream_t s, const uint32_t* tokp, bool h16) {
  ProjArgs a{};
  a.w = w;
  a.k = k;
  a.ss = ss;
  a.caches = caches;
  a.cache_stride = cache_stride;
  a.logits = logits;
  a.capture = nullptr;
  a.tokp = tokp;
  a.sb = ss.B == 1 ? 1 : BATCH_SB;
  if (h16) {
    if (ss.B != 1) return hipErrorInvalidValue;
    launch_layers<2, 1, 1, true>(a, s);
  } else if (ss.B == 1) {
    launch_layers<2, 1, 1, false>(a, s);
  } else {
    a.preln = BATCH_PRELN;
    launch_layers<BATCH_RPW, BATCH_BT768, BATCH_BT3072, false, BATCH_RPW_PR>(a, s);
  }
  return hipGetLastError();
}

template <int MODE, int RPW>
static void launch_q8(const ProjArgs& a, hipStream_t s) {
  const int rows = MODE == MODE_QKV ? D3 : MODE == MODE_FC ? F : MODE == MODE_HEAD ? V : D;
  constexpr int NW = q8_waves(MODE);
  const int nblk = (rows + NW * RPW - 1) / (NW * RPW);
  hipLaunchKernelGGL((k_q8proj<MODE, RPW>), dim3(nblk), dim3(64 * NW), 0, s, a);
}

hipError_t launch_step_q8(const Weights& w, const Work& k, const Sessions& ss, float* cache,
                          float* logits, char* capture, hipStream_t s, const uint32_t* tokp, int qx, int qw) {
  ProjArgs a{};
  a.w = w;
  a.k = k;
  a.ss = ss;
  a.caches = cache;
  a.cache_stride = 0;
  a.logits = logits;
  a.capture = capture;
  a.qx = qx;
  a.qw = qw;
  a.sb = 1;
  hipLaunchKernelGGL(k_embed, dim3(1), dim3(192), 0, s, w, ss, k.x, tokp);
  for (int l = 0; l < L; ++l) {
    a.layer = l;
    launch_q8<MODE_QKV, 2>(a, s);
    hipLaunchKernelGGL(k_attn<true>, dim3(H, 1), dim3(attn_threads<true>()), 0, s, a);
    launch_q8<MODE_O, 1>(a, s);
    launch_q8<MODE_FC, 2>(a, s);
    launch_q8<MODE_PR, 1>(a, s);
  }
  launch_q8<MODE_HEAD, 4>(a, s);
  return hipGetLastError();
}

// Final LayerNorm and tied head of one residual row (used by the full-prefix path).
hipError_t launch_head_f32(const Weights& w, const float* x_row, float* logits, hipStream_t s) {
  ProjArgs a{};
  a.w = w;
  a.k.x = const_cast<float*>(x_row);
  a.ss.B = 1;
  a.sb = 1;
  a.logits = logits;
  launch_proj<MODE_HEAD, 2, 1, false>(a, s);
  return hipGetLastError();
}

hipError_t launch_special_bits(int kind, uint32_t first, long long n, float* y, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_special_bits, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, kind, first, n, y);
  return hipGetLastError();
}

hipError_t launch_layernorm_seq(const float* x, int rows, const float* gamma, const float* beta, float* y,
                                hipStream_t s) {
  if (rows > 0) hipLaunchKernelGGL(k_layernorm_seq, dim3(rows), dim3(512), 0, s, x, gamma, beta, y);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, uint32_t* next, uint32_t* tokens_out, int32_t* status, int step,
                         hipStream_t s) {
  hipLaunchKernelGGL(k_argmax, dim3(1), dim3(1024), 0, s, logits, next, tokens_out, status, step);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* x, int n, int8_t* codes, float* scales, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_quantize, dim3(n / 64), dim3(64), 0, s, x, codes, scales);
  return hipGetLastError();
}

}  // namespace g2
