// Fused single-launch decode step (batch 1): one token through the 12 blocks and
// the tied head (LeanExe GPT-2 README, cachedStep paragraph) in one cooperative
// launch of one 512-thread workgroup per compute unit.
//
// Why: a step is ~61 dependent phases over ~495 MB (fp32) or ~137 MB (int8) of
// weights; launching a kernel per phase costs ~1.7-2.5 us each on MI355X, more than
// the phase's own HBM time.  Here the weights of every phase of block l+1 are
// loaded into registers while block l computes (each compute wave owns at most
// one output row per phase), so the weight stream is decoupled from the chain of
// cross-workgroup exchanges, and each exchange costs about one memory round trip.
//
// Roles inside the grid (workgroups of 8 waves):
//  - workgroups 0..11 run attention, one head each, with the head's key/value
//    rows staged in LDS;
//  - the other workgroups own the projection rows: compute wave c of C (global
//    index) owns rows c, c + C, ... of every projection (at most 2 QKV, 1 O, 3 FC,
//    1 PR rows per block), and every workgroup takes rows of the tied head at the end;
//  - wave 0 of each workgroup receives the phase input and hands it to the
//    compute waves through LDS and s_barrier (no vmcnt drain, so register
//    prefetches stay in flight); wave 1 stages the next block's LayerNorm
//    parameters in LDS.
//
// Exchanges carry (value, epoch) 64-bit words: a producer stores value and epoch
// in one agent-scope store, a consumer polls until every word has this launch's
// epoch, so no fence or flag is needed.  Vectors every workgroup needs (attention
// output, x1, GELU output, x2) are written by their producers into one copy per
// XCD (eight lanes store the eight copies in one instruction), and each
// workgroup's input wave polls its own XCD's copy: this spreads the polling over
// eight sets of memory lines.  The epoch advances once per launch (header word 0),
// written by the last workgroup to finish.  Every wait is bounded: past
// SPIN_LIMIT polls a workgroup records an error code in header word 2, every
// other wait then returns at once, and the launch runs to its end.
//
// Every output value is computed by the same device functions as the per-phase
// kernels (layernorm_frag / dot_frag / attn_compute / gelu_tanh for fp32;
// layernorm_seq / quant_lane / q8_dot for int8), so the fused step gives the same
// bits as the per-phase path and as the batched step.
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace g2 {

typedef unsigned long long u64;

constexpr int FT = 512;           // threads per workgroup (8 waves: input, parameters, 6 compute)
constexpr int NCW = FT / 64 - 2;  // compute waves per workgroup
constexpr int MIN_GRID = 204;     // smallest grid for which the row bounds below hold
// Rows of each projection per compute wave (rows r = c + k * compute_waves).
constexpr int RPW_QKV = 2, RPW_O = 1, RPW_FC = 3, RPW_PR = 1;
constexpr int HEAD_MAX_ROWS = 42;  // ceil(V / (NCW * MIN_GRID))
constexpr int NATT = H;           // attention workgroups
constexpr unsigned SPIN_LIMIT = 1u << 21;

// Global exchange words per block: qkv | att | x1 | g | x2.
constexpr int LO_QKV = 0, LO_ATT = D3, LO_X1 = D3 + D, LO_G = D3 + 2 * D, LO_X2 = D3 + 2 * D + F;
static_assert(LO_X2 + D == LL_PER_LAYER, "exchange layout");
// Per-XCD copies per block: att | x1 | g | x2.
constexpr int RO_ATT = 0, RO_X1 = D, RO_G = 2 * D, RO_X2 = 2 * D + F;
static_assert(RO_X2 + D == L2_PER_LAYER, "copy layout");
constexpr int NXCC = 8;  // XCDs of an MI355X in single-partition mode

enum { HDR_EPOCH = 0, HDR_DONE = 1, HDR_ERROR = 2 };
enum { ERR_SPIN = 1, ERR_XCC = 2 };

struct FusedArgs {
  Weights w;
  float* cache;
  float* logits;
  u64* ll;           // [L][LL_PER_LAYER]: qkv words (one copy, read by attention)
  u64* l2;           // [NXCC][L][L2_PER_LAYER]: per-XCD copies of att, x1, g, x2
  uint32_t* header;
  char* capture;     // int8 test capture or null
  uint64_t* trace;   // timeline test hook or null: [grid][64] timestamps
  uint32_t token;
  int32_t pos;
};

// Timeline test hook: slot 0 kernel start; 1+4l+{0..3} inputs of QKV/O/FC/PR of block l
// received (projection workgroups) or 1+4l+{0,1} qkv received / attention done
// (attention workgroups); 49 head input received; 50 head rows done; 51 end.
__device__ __forceinline__ void stamp(const uint64_t* trace, int slot) {
  if (trace) ((uint64_t*)trace)[blockIdx.x * 64 + slot] = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ u64 ld_sc1(const u64* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_sc1(u64* p, u64 v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ uint32_t ld32(const uint32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ u64 pack(float v, uint32_t e) { return ((u64)e << 32) | __float_as_uint(v); }
__device__ __forceinline__ uint32_t epoch_of(u64 w) { return (uint32_t)(w >> 32); }

// Workgroup barrier that waits only for this wave's LDS traffic, not for its
// outstanding global loads (register prefetches stay in flight across it).
__device__ __forceinline__ void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xf;
}

__device__ __forceinline__ void set_error(uint32_t* header, uint32_t code) { atomicCAS(&header[HDR_ERROR], 0u, code); }

// Bounded-wait bookkeeping: true when the wait must stop (limit reached or
// another workgroup already failed).
__device__ __forceinline__ bool give_up(uint32_t& spins, uint32_t* header) {
  if ((++spins & 127) != 0) return false;
  if (spins > SPIN_LIMIT) {
    set_error(header, ERR_SPIN);
    return true;
  }
  return ld32(&header[HDR_ERROR]) != 0;
}

// One wave polls PL*64 global words at src[lane + 64j] until all carry epoch E.
template <int PL>
__device__ __forceinline__ bool poll_global(const u64* src, uint32_t E, u64 (&w)[PL], uint32_t* header) {
  const int lane = lane_id();
  uint32_t spins = 0;
  while (true) {
#pragma unroll
    for (int j = 0; j < PL; ++j) w[j] = ld_sc1(src + lane + 64 * j);
    bool ok = true;
#pragma unroll
    for (int j = 0; j < PL; ++j) ok &= epoch_of(w[j]) == E;
    if (__all(ok)) return true;
    if (give_up(spins, header)) return false;
  }
}

// Input wave: poll this XCD's copy of a PL*64-word vector until every word has
// epoch E, then write the values to LDS (and optionally a second LDS copy).
template <int PL>
__device__ __forceinline__ void receive(const u64* src, uint32_t E, float* out, float* out2, uint32_t* header) {
  const int lane = lane_id();
  u64 w[PL];
  poll_global<PL>(src, E, w, header);
#pragma unroll
  for (int j = 0; j < PL; ++j) {
    const float v = __uint_as_float((uint32_t)w[j]);
    out[lane + 64 * j] = v;
    if (out2) out2[lane + 64 * j] = v;
  }
}

// Producer side of a per-XCD vector: lanes 0..NXCC-1 of the producing wave store
// word idx of block l's slice `off` into every XCD's copy.
__device__ __forceinline__ void publish(u64* l2, int l, int off, int idx, float v, uint32_t E) {
  const int lane = lane_id();
  if (lane < NXCC) st_sc1(l2 + ((size_t)lane * L + l) * L2_PER_LAYER + off + idx, pack(v, E));
}

// ---- per-wave weight registers ----------------------------------------------
// fp32: 30 slots of one float4 per lane.  A 768-input row takes 3 slots, a
// 3072-input row 12: QKV rows k=0,1 -> slots 0-5, O -> 6-8, FC k=0..2 -> 9-17,
// PR -> 18-29.  For the head, slots 3s..3s+2 hold head row slot s (10 slots).
// int8: 9 slots of one int4 per lane (a 768-input row takes 1, a 3072-input row 3):
// QKV 0-1, O 2, FC 3-5, PR 6-8; head rows use slots 0-8.  sc[] is the lane-g
// weight scale of the row whose first slot it indexes.
template <bool Q8>
struct WRegs;
template <>
struct WRegs<false> {
  f4 r[30];
  float b[7];  // bias of QKV k=0,1, O, FC k=0..2, PR
};
template <>
struct WRegs<true> {
  i4 c[9];
  float sc[9];
  float b[7];
};

constexpr int f32_slot(int m, int k) { return m == M_QKV ? 3 * k : m == M_O ? 6 : m == M_FC ? 9 + 3 * k : 18; }
constexpr int q8_slot(int m, int k) { return m == M_QKV ? k : m == M_O ? 2 : m == M_FC ? 3 + k : 6; }
constexpr int bias_slot(int m, int k) { return m == M_QKV ? k : m == M_O ? 2 : m == M_FC ? 3 + k : 6; }
constexpr int rpw(int m) { return m == M_QKV ? RPW_QKV : m == M_O ? RPW_O : m == M_FC ? RPW_FC : RPW_PR; }

// Row k of matrix m (block l) owned by compute wave c of C, into its slots.
template <bool Q8, int m, int k>
__device__ __forceinline__ void load_row(WRegs<Q8>& R, const Weights& w, int l, int c, int C) {
  const int r = c + k * C;
  if (r >= mat_rows(m)) return;
  const int lane = lane_id();
  const int bofs = m == M_QKV ? sp::B_QKV : m == M_O ? sp::B_O : m == M_FC ? sp::B_FC : sp::B_PR;
  if constexpr (!Q8) {
    const float* W = f32_mat(w, l, m) + (size_t)r * mat_cols(m);
    constexpr int s0 = f32_slot(m, k), n = mat_cols(m) / 256;
#pragma unroll
    for (int i = 0; i < n; ++i) R.r[s0 + i] = __builtin_nontemporal_load((const f4*)(W + 256 * i + 4 * lane));
  } else {
    constexpr int s0 = q8_slot(m, k);
    if constexpr (m == M_PR) {
      i4 t[3];
      q8_load_row<F>(t, R.sc[s0], q8_codes(w, l, m), q8_scales(w, l, m), r);
      R.c[s0] = t[0]; R.c[s0 + 1] = t[1]; R.c[s0 + 2] = t[2];
    } else {
      i4 t[1];
      q8_load_row<D>(t, R.sc[s0], q8_codes(w, l, m), q8_scales(w, l, m), r);
      R.c[s0] = t[0];
    }
  }
  R.b[bias_slot(m, k)] = small_p(w, l, bofs)[r];
}

template <bool Q8>
constexpr int head_slots() { return Q8 ? 9 : 10; }

// Head row r into head slot s.
template <bool Q8>
__device__ __forceinline__ void load_head(WRegs<Q8>& R, const Weights& w, int s, int r) {
  if (r >= V) return;
  if constexpr (!Q8) {
    const int lane = lane_id();
    const float* row = w.wte + (size_t)r * D;
#pragma unroll
    for (int i = 0; i < 3; ++i) R.r[3 * s + i] = __builtin_nontemporal_load((const f4*)(row + 256 * i + 4 * lane));
  } else {
    i4 t[1];
    q8_load_row<D>(t, R.sc[s], q8_codes(w, 0, M_HEAD), q8_scales(w, 0, M_HEAD), r);
    R.c[s] = t[0];
  }
}

// int8: quantize the K-vector src (LDS) into codes/scales (LDS), groups spread over
// the compute waves.
__device__ __forceinline__ void quantize_input(const float* src, int K, int8_t* xc, float* xsc, int wave) {
  const int lane = lane_id();
  for (int g = wave - 2; g < K / 64; g += NCW) {
    float s;
    const int c = quant_lane(src[g * 64 + lane], s);
    xc[g * 64 + lane] = (int8_t)c;
    if (lane == 0) xsc[g] = s;
  }
}

// The io wave overwrites an input buffer only once every reader of the previous
// contents has produced its output (that output is part of the new input), so one
// buffer per input suffices, except for the 3072-word GELU vector, which arrives in
// four pieces while FC rows may still be reading x1: it has its own buffer xg.
struct FusedSmem {
  float xs[D];      // input of QKV (x), O (attention output), FC (x1), head (x2)
  float xg[F];      // input of PR (GELU output)
  float xres[D];    // residual of the current sub-block
  float xn[D];      // int8 path: LayerNorm output
  float lnp[2][4][D];  // LayerNorm parameters by block parity: ln1 gamma, beta, ln2 gamma, beta
  float lnf[2][D];     // final LayerNorm gamma, beta
  int8_t xc[F];     // int8 path: input codes
  float xsc[64];    // int8 path: input scales
  AttnSmem att;     // attention workgroups
};

// Per-workgroup constants shared by the wave roles.
struct Ctx {
  uint32_t E;          // this launch's epoch
  int xcc;             // XCD of this workgroup
  u64* cp;             // this XCD's copies
  int G;               // workgroups in the grid
};

__device__ __forceinline__ const u64* copy_of(const Ctx& c, int l, int off) {
  return c.cp + (size_t)l * L2_PER_LAYER + off;
}

// Wave 1: copy a 768-vector from global memory into LDS.
__device__ __forceinline__ void stage_vec(float* dst, const float* src) {
  const int lane = lane_id();
  f4 v[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) v[i] = *(const f4*)(src + 256 * i + 4 * lane);
#pragma unroll
  for (int i = 0; i < 3; ++i) *(f4*)(dst + 256 * i + 4 * lane) = v[i];
}
__device__ __forceinline__ void stage_ln(FusedSmem& S, const Weights& w, int l) {
  float (*p)[D] = S.lnp[l & 1];
  stage_vec(p[0], small_p(w, l, sp::LN1_G));
  stage_vec(p[1], small_p(w, l, sp::LN1_B));
  stage_vec(p[2], small_p(w, l, sp::LN2_G));
  stage_vec(p[3], small_p(w, l, sp::LN2_B));
}

// ---- projection workgroups: waves 0 and 1 --------------------------------------
// Per phase: wave 0 polls its XCD's copy of the phase input and puts it in LDS (on
// the int8 path also the sequential LayerNorm of it); then barrier B1.  Wave 1
// stages block l+1's LayerNorm parameters during block l.  On the int8 path the
// compute waves quantize between B1 and B2; waves 0-1 write the capture of the
// input side (test hook) after B2.
template <bool Q8>
__device__ void io_waves(const FusedArgs a, FusedSmem& S, const Ctx c) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint32_t* hdr = a.header;
  char* cap = (Q8 && a.capture && (int)blockIdx.x == NATT) ? a.capture : nullptr;
  auto after_b1 = [&](int l, int m, const float* x) {
    if constexpr (Q8) {
      wg_barrier();  // B2: codes ready
      if (cap) {
        const CapLayout cl = cap_item(m);
        char* base = cap + cap_offset(l, m);
        const int K = mat_cols(m);
        for (int i = (int)threadIdx.x; i < K; i += 128) {
          ((float*)(base + cl.in))[i] = x[i];
          ((int8_t*)(base + cl.codes))[i] = S.xc[i];
        }
        if ((int)threadIdx.x < K / 64) ((float*)(base + cl.xs))[threadIdx.x] = S.xsc[threadIdx.x];
      }
    }
  };
  if (wave == 1) {
    stage_ln(S, a.w, 0);
    stage_vec(S.lnf[0], a.w.small + sp::LNF_G);
    stage_vec(S.lnf[1], a.w.small + sp::LNF_B);
  }
  wg_barrier();  // B0: block 0's LayerNorm parameters are in LDS
  for (int l = 0; l < L; ++l) {
    const float(*lp)[D] = S.lnp[l & 1];
    // QKV input: the embedding at block 0, else the previous block's x2
    if (wave == 0) {
      if (l == 0) {
#pragma unroll
        for (int j = 0; j < 12; ++j) {
          const int i = lane + 64 * j;
          const float v = a.w.wte[(size_t)a.token * D + i] + a.w.wpe[(size_t)a.pos * D + i];
          S.xs[i] = v;
          S.xres[i] = v;
        }
      } else {
        receive<12>(copy_of(c, l - 1, RO_X2), c.E, S.xs, S.xres, hdr);
      }
      if (lane == 0) stamp(a.trace, 1 + 4 * l);
      if constexpr (Q8) layernorm_seq(S.xs, lp[0], lp[1], S.xn);
    }
    wg_barrier();  // B1
    after_b1(l, M_QKV, S.xn);
    if (wave == 1 && l + 1 < L) stage_ln(S, a.w, l + 1);
    // O input: attention output
    if (wave == 0) {
      receive<12>(copy_of(c, l, RO_ATT), c.E, S.xs, nullptr, hdr);
      if (lane == 0) stamp(a.trace, 2 + 4 * l);
    }
    wg_barrier();
    after_b1(l, M_O, S.xs);
    // FC input: x1
    if (wave == 0) {
      receive<12>(copy_of(c, l, RO_X1), c.E, S.xs, S.xres, hdr);
      if (lane == 0) stamp(a.trace, 3 + 4 * l);
      if constexpr (Q8) layernorm_seq(S.xs, lp[2], lp[3], S.xn);
    }
    wg_barrier();
    after_b1(l, M_FC, S.xn);
    // PR input: GELU output
    if (wave == 0) {
      receive<48>(copy_of(c, l, RO_G), c.E, S.xg, nullptr, hdr);
      if (lane == 0) stamp(a.trace, 4 + 4 * l);
    }
    wg_barrier();
    after_b1(l, M_PR, S.xg);
  }
  // head input
  if (wave == 0) {
    receive<12>(copy_of(c, L - 1, RO_X2), c.E, S.xs, nullptr, hdr);
    if (lane == 0) stamp(a.trace, 49);
    if constexpr (Q8) layernorm_seq(S.xs, S.lnf[0], S.lnf[1], S.xn);
  }
  wg_barrier();
  after_b1(0, M_HEAD, S.xn);
}

// Head rows of wave hw (rows hw + k*hstride): slots were loaded ahead; each slot is
// refilled with the row NS further on as soon as it has been used.
template <bool Q8>
__device__ __forceinline__ void head_rows(const FusedArgs a, FusedSmem& S, WRegs<Q8>& R, int hw, int hstride) {
  const int lane = lane_id();
  char* capr = Q8 ? a.capture : nullptr;
  f4 x[3];
  if constexpr (!Q8) {
    load_frag<3>(x, S.xs);
    layernorm_frag(x, S.lnf[0], S.lnf[1]);
  }
  constexpr int NS = head_slots<Q8>();
  const int nrows = (V - hw + hstride - 1) / hstride;
#pragma unroll
  for (int k = 0; k < HEAD_MAX_ROWS; ++k) {
    // keep the loads in slot order: at most NS rows in flight per wave
    __builtin_amdgcn_sched_barrier(0);
    if (k >= nrows) continue;
    const int r = hw + k * hstride;
    const int s = k % NS;
    float y;
    if constexpr (!Q8) {
      y = dot_frag<3>(*reinterpret_cast<f4(*)[3]>(&R.r[3 * s]), x);
    } else {
      int32_t* ca = capr ? (int32_t*)(capr + cap_offset(0, M_HEAD) + cap_item(M_HEAD).acc) + (size_t)r * 12 : nullptr;
      y = q8_dot<D>(*reinterpret_cast<i4(*)[1]>(&R.c[s]), R.sc[s], S.xc, S.xsc, ca);
      if (capr && lane == 0) ((float*)(capr + cap_offset(0, M_HEAD) + cap_item(M_HEAD).y))[r] = y;
    }
    if (lane == 0) a.logits[r] = y;
    load_head<Q8>(R, a.w, s, r + NS * hstride);
  }
}

// ---- projection workgroups: compute waves 2..7 ---------------------------------
template <bool Q8>
__device__ void compute_waves(const FusedArgs a, FusedSmem& S, const Ctx c) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int npw = c.G - NATT;
  const int C = NCW * npw;                                      // compute waves of the grid
  const int cw = (wave - 2) * npw + ((int)blockIdx.x - NATT);  // this wave's index
  const int hw = (wave - 2) * c.G + (int)blockIdx.x;            // first head row
  const int hstride = NCW * c.G;
  const uint32_t E = c.E;
  char* capr = Q8 ? a.capture : nullptr;
  auto quantize = [&](const float* src, int K) {
    if constexpr (Q8) {
      quantize_input(src, K, S.xc, S.xsc, wave);
      wg_barrier();  // B2
    }
  };
  // y = projection row k of matrix m at block l (bias included), for the input in LDS
  auto project = [&](WRegs<Q8>& R, int l, auto mc, auto kc, int r) -> float {
    constexpr int m = decltype(mc)::value, k = decltype(kc)::value;
    float y;
    if constexpr (!Q8) {
      constexpr int s0 = f32_slot(m, k);
      if constexpr (m == M_PR) {
        y = dot_lds<12>(*reinterpret_cast<f4(*)[12]>(&R.r[s0]), S.xg);
      } else {
        f4 x[3];
        load_frag<3>(x, S.xs);
        if constexpr (m == M_QKV) layernorm_frag(x, S.lnp[l & 1][0], S.lnp[l & 1][1]);
        if constexpr (m == M_FC) layernorm_frag(x, S.lnp[l & 1][2], S.lnp[l & 1][3]);
        y = dot_frag<3>(*reinterpret_cast<f4(*)[3]>(&R.r[s0]), x);
      }
    } else {
      constexpr int s0 = q8_slot(m, k);
      int32_t* ca = capr ? (int32_t*)(capr + cap_offset(l, m) + cap_item(m).acc) + (size_t)r * (mat_cols(m) / 64) : nullptr;
      if constexpr (m == M_PR) y = q8_dot<F>(*reinterpret_cast<i4(*)[3]>(&R.c[s0]), R.sc[s0], S.xc, S.xsc, ca);
      else y = q8_dot<D>(*reinterpret_cast<i4(*)[1]>(&R.c[s0]), R.sc[s0], S.xc, S.xsc, ca);
    }
    y = y + R.b[bias_slot(m, k)];
    if (Q8 && capr && lane == 0) ((float*)(capr + cap_offset(l, m) + cap_item(m).y))[r] = y;
    return y;
  };
  using QKVm = std::integral_constant<int, M_QKV>;
  using Om = std::integral_constant<int, M_O>;
  using FCm = std::integral_constant<int, M_FC>;
  using PRm = std::integral_constant<int, M_PR>;
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using K2 = std::integral_constant<int, 2>;

  WRegs<Q8> R;
  load_row<Q8, M_QKV, 0>(R, a.w, 0, cw, C);
  load_row<Q8, M_QKV, 1>(R, a.w, 0, cw, C);
  load_row<Q8, M_O, 0>(R, a.w, 0, cw, C);
  load_row<Q8, M_FC, 0>(R, a.w, 0, cw, C);
  load_row<Q8, M_FC, 1>(R, a.w, 0, cw, C);
  load_row<Q8, M_FC, 2>(R, a.w, 0, cw, C);
  load_row<Q8, M_PR, 0>(R, a.w, 0, cw, C);
  wg_barrier();  // B0

  for (int l = 0; l < L; ++l) {
    u64* gl = a.ll + (size_t)l * LL_PER_LAYER;
    const bool last = l + 1 == L;
    // QKV: rows also append the key/value row of this position to the cache
    wg_barrier();
    quantize(S.xn, D);
    auto qkv_row = [&](auto kc) {
      const int r = cw + decltype(kc)::value * C;
      if (r < D3) {
        const float y = project(R, l, QKVm{}, kc, r);
        if (lane == 0) {
          st_sc1(gl + LO_QKV + r, pack(y, E));
          if (r >= D) a.cache[((size_t)a.pos * L + l) * KV_ROW + (r - D)] = y;
        }
      }
      if (!last) load_row<Q8, M_QKV, decltype(kc)::value>(R, a.w, l + 1, cw, C);
    };
    qkv_row(K0{});
    qkv_row(K1{});
    // O: residual add into x1
    wg_barrier();
    quantize(S.xs, D);
    {
      const int r = cw;
      if (r < D) {
        const float y = project(R, l, Om{}, K0{}, r);
        publish(a.l2, l, RO_X1, r, S.xres[r] + y, E);
      }
      if (!last) load_row<Q8, M_O, 0>(R, a.w, l + 1, cw, C);
    }
    // FC: GELU
    wg_barrier();
    quantize(S.xn, D);
    auto fc_row = [&](auto kc) {
      const int r = cw + decltype(kc)::value * C;
      if (r < F) {
        const float y = project(R, l, FCm{}, kc, r);
        publish(a.l2, l, RO_G, r, gelu_tanh(y), E);
      }
      if (!last) load_row<Q8, M_FC, decltype(kc)::value>(R, a.w, l + 1, cw, C);
    };
    fc_row(K0{});
    fc_row(K1{});
    fc_row(K2{});
    // PR: residual add into x2
    wg_barrier();
    quantize(S.xg, F);
    {
      const int r = cw;
      if (r < D) {
        const float y = project(R, l, PRm{}, K0{}, r);
        publish(a.l2, l, RO_X2, r, S.xres[r] + y, E);
      }
      if (!last) load_row<Q8, M_PR, 0>(R, a.w, l + 1, cw, C);
    }
  }
  // all slots are free after the last block: start the head rows
#pragma unroll
  for (int s = 0; s < head_slots<Q8>(); ++s) load_head<Q8>(R, a.w, s, hw + s * hstride);
  wg_barrier();
  quantize(S.xn, D);
  head_rows<Q8>(a, S, R, hw, hstride);
  if (wave == 2 && lane == 0) stamp(a.trace, 50);
}

// ---- attention workgroups (head h = blockIdx.x) --------------------------------
template <bool Q8>
__device__ void attention_wg(const FusedArgs a, FusedSmem& S, const Ctx c) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int h = blockIdx.x, pos = a.pos;
  uint32_t* hdr = a.header;
  AttnSmem& sm = S.att;
  if (wave == 1) {
    stage_vec(S.lnf[0], a.w.small + sp::LNF_G);
    stage_vec(S.lnf[1], a.w.small + sp::LNF_B);
  }
  for (int l = 0; l < L; ++l) {
    const u64* gl = a.ll + (size_t)l * LL_PER_LAYER;
    const float* cl = a.cache + (size_t)l * KV_ROW + h * DH;
    auto kv = [&](int j) { return cl + (size_t)j * CACHE_POS; };
    attn_stage_rows(sm, kv, 0, pos, 64, FT - 64);
    if (wave == 0) {
      u64 w0, w1, w2;
      uint32_t spins = 0;
      while (true) {
        w0 = ld_sc1(gl + LO_QKV + h * DH + lane);
        w1 = ld_sc1(gl + LO_QKV + D + h * DH + lane);
        w2 = ld_sc1(gl + LO_QKV + 2 * D + h * DH + lane);
        if (__all(epoch_of(w0) == c.E && epoch_of(w1) == c.E && epoch_of(w2) == c.E)) break;
        if (give_up(spins, hdr)) break;
      }
      if (lane == 0) stamp(a.trace, 1 + 4 * l);
      sm.q[lane] = __uint_as_float((uint32_t)w0);
      sm.k[pos][lane] = __uint_as_float((uint32_t)w1);
      sm.v[pos][lane] = __uint_as_float((uint32_t)w2);
    }
    __syncthreads();
    const float o = attn_compute(sm, pos + 1);
    if (wave == 0) {
#pragma unroll
      for (int x = 0; x < NXCC; ++x)
        st_sc1(a.l2 + ((size_t)x * L + l) * L2_PER_LAYER + RO_ATT + h * DH + lane, pack(o, c.E));
      if (lane == 0) stamp(a.trace, 2 + 4 * l);
    }
    __syncthreads();
  }
  // the tied head: these workgroups take head rows too
  const int hw = (wave - 2) * c.G + (int)blockIdx.x;
  const int hstride = NCW * c.G;
  if (wave == 0) {
    receive<12>(copy_of(c, L - 1, RO_X2), c.E, S.xs, nullptr, hdr);
    if constexpr (Q8) layernorm_seq(S.xs, S.lnf[0], S.lnf[1], S.xn);
    wg_barrier();
    if constexpr (Q8) wg_barrier();
  } else if (wave == 1) {
    wg_barrier();
    if constexpr (Q8) wg_barrier();
  } else {
    WRegs<Q8> R;
#pragma unroll
    for (int s = 0; s < head_slots<Q8>(); ++s) load_head<Q8>(R, a.w, s, hw + s * hstride);
    wg_barrier();
    if constexpr (Q8) {
      quantize_input(S.xn, D, S.xc, S.xsc, wave);
      wg_barrier();
    }
    head_rows<Q8>(a, S, R, hw, hstride);
  }
}

template <bool Q8>
__global__ __launch_bounds__(FT, 1) void k_fused(const FusedArgs a) {
  extern __shared__ __align__(16) char smem_raw[];
  FusedSmem& S = *(FusedSmem*)smem_raw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t* hdr = a.header;
  if (threadIdx.x == 0) stamp(a.trace, 0);
  Ctx c;
  c.E = ld32(&hdr[HDR_EPOCH]) + 1u;
  c.xcc = (int)xcc_id();
  if (c.xcc >= NXCC) {
    if (threadIdx.x == 0) set_error(hdr, ERR_XCC);
    c.xcc = 0;
  }
  c.cp = a.l2 + (size_t)c.xcc * L * L2_PER_LAYER;
  c.G = gridDim.x;
  if ((int)blockIdx.x < NATT) attention_wg<Q8>(a, S, c);
  else if (wave < 2) io_waves<Q8>(a, S, c);
  else compute_waves<Q8>(a, S, c);

  __syncthreads();
  if (threadIdx.x == 0) {
    stamp(a.trace, 51);
    const uint32_t done = atomicAdd(&hdr[HDR_DONE], 1u);
    if (done == (uint32_t)c.G - 1) {
      hdr[HDR_DONE] = 0;
      __hip_atomic_store(&hdr[HDR_EPOCH], c.E, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---- host side ---------------------------------------------------------------

struct FusedConfig {
  int ok;    // 1 usable, 0 not yet probed, -1 unusable (fall back to per-phase kernels)
  int grid;
};
static FusedConfig g_cfg[2][64];
uint64_t* g_fused_trace = nullptr;  // timeline test hook
int g_fused_plain_launch = 1;       // 1: ordinary launch (default), 0: cooperative launch

template <bool Q8>
static hipError_t fused_config(FusedConfig& c) {
  if (c.ok) return hipSuccess;
  int dev = 0, cus = 0, coop = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev))) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev))) return e;
  if ((e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev))) return e;
  const size_t lds = sizeof(FusedSmem);
  if ((e = hipFuncSetAttribute((const void*)k_fused<Q8>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)))
    return e;
  int per_cu = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_fused<Q8>, FT, lds))) return e;
  // The per-wave row bounds (RPW_*, HEAD_MAX_ROWS) need at least MIN_GRID workgroups.
  const bool enough = cus >= MIN_GRID && cus <= 4096;
  c.grid = cus;
  c.ok = (coop && per_cu >= 1 && enough) ? 1 : -1;
  return hipSuccess;
}

template <bool Q8>
static hipError_t launch_fused_t(const Weights& w, const Work& k, uint32_t token, int32_t pos, float* cache,
                                 float* logits, char* capture, hipStream_t s, bool* used) {
  *used = false;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e) return e;
  FusedConfig& c = g_cfg[Q8 ? 1 : 0][dev & 63];
  if ((e = fused_config<Q8>(c))) return e;
  if (c.ok != 1) return hipSuccess;
  FusedArgs a{};
  a.w = w;
  a.cache = cache;
  a.logits = logits;
  a.ll = k.ll;
  a.l2 = k.ll + (size_t)L * LL_PER_LAYER;
  a.header = k.header;
  a.capture = capture;
  a.trace = g_fused_trace;
  a.token = token;
  a.pos = pos;
  void* args[] = {&a};
  if (g_fused_plain_launch)
    e = hipLaunchKernel((const void*)k_fused<Q8>, dim3(c.grid), dim3(FT), args, sizeof(FusedSmem), s);
  else
    e = hipLaunchCooperativeKernel((const void*)k_fused<Q8>, dim3(c.grid), dim3(FT), args, sizeof(FusedSmem), s);
  if (e == hipSuccess) *used = true;
  return e;
}

hipError_t launch_fused(bool q8, const Weights& w, const Work& k, uint32_t token, int32_t pos, float* cache,
                        float* logits, char* capture, hipStream_t s, bool* used) {
  return q8 ? launch_fused_t<true>(w, k, token, pos, cache, logits, capture, s, used)
            : launch_fused_t<false>(w, k, token, pos, cache, logits, capture, s, used);
}

}  // namespace g2
