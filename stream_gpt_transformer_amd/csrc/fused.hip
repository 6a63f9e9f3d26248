// Fused single-launch decode step (batch 1): one token through the 12 blocks and
// the tied head (LeanExe GPT-2 README, cachedStep paragraph) in one launch of one
// 512-thread workgroup per compute unit.
//
// Why one launch: a step is a chain of ~60 dependent phases over ~495 MB (fp32) or
// ~137 MB (int8) of weights; a kernel launch per phase costs ~1.7-2.5 us on MI355X,
// more than most phases' own HBM time.  Here every compute wave holds the weights
// of its share of block l+1 in registers while block l runs, so the weight stream
// is decoupled from the chain of exchanges between workgroups.
//
// Placement: the eight XCDs are used like eight tensor-parallel devices, each with
// its own L2.  Workgroup b runs on XCD b % 8 (the dispatcher deals workgroups
// round-robin over the XCDs; every launch checks it) with rank b / 8 in it.  XCD X
// owns heads X and X + 8 (when below 12), the FC rows 384X..384X+383 and the
// matching 384-input slice of the MLP projection.  Ranks 0 and 1 run the
// attention of the XCD's heads (K/V rows staged in LDS); ranks 2..31 compute:
//  - inside the XCD (through its L2: plain stores, non-temporal polls) travel the
//    q/k/v and attention outputs of its heads, its GELU slice, and the
//    all-gathers of x1 and x2;
//  - the two sums over all XCDs of a block are reduce-scatters through device
//    memory: the XCDs publish terms (output projection: one per head; MLP
//    projection: one per slice for fp32, one per 64-group for int8), every
//    workgroup polls the terms of its 24 outputs, adds them in fixed order plus
//    bias and residual, and writes the 24 values into its XCD's copy of x1/x2.
// Each block thus has two exchanges across XCDs and five inside one.
//
// Waves of a compute workgroup: wave 0 receives (polls, reduce-scatters,
// all-gathers, the int8 LayerNorm) and stages the next block's LayerNorm
// parameters while it waits; waves 1..7 compute.  Compute wave c of an XCD's 210
// owns at most two units of every phase (QKV rows, head-group dots of the output
// projection, FC rows, slice dots of the MLP projection) and holds their weights
// in registers.
//
// Exchange words are (epoch << 32 | value bits), stored with one 64-bit store, so
// a poll that sees this launch's epoch sees the value: no flags, no fences.  The
// epoch advances once per launch (header word 0, written by the last workgroup to
// finish).  Every wait is bounded: past SPIN_LIMIT polls a workgroup records an
// error in header word 2, every other wait then returns at once, and the launch
// runs to its end.
//
// Arithmetic: QKV/FC rows, the head, attention, LayerNorm and GELU use the device
// functions shared with the per-phase kernels; the output projection is
// y = 0, y = y + p_h over the 12 heads, the fp32 MLP projection y = 0, y = y + p_s
// over 8 slices (o_row / pr_row give the same bits), the int8 MLP projection
// y = 0, y = y + t_g over its 48 groups (as q8_dot).  So the fused step, the
// per-phase kernels and the batched step give the same bits, and the int8 step
// the oracle's.
#include <type_traits>

#include "device.hpp"
#include "internal.hpp"

namespace g2 {

typedef unsigned long long u64;

constexpr int FT = 512;               // threads per workgroup
constexpr int NX = FX_NXCC;           // XCDs
constexpr int NR = 32;                // workgroups per XCD
constexpr int GRID = NX * NR;         // 256 = compute units of an MI355X
constexpr int NCW = 7;                // compute waves per workgroup (waves 1..7)
constexpr int CR0 = 2;                // first compute rank
constexpr int CW = (NR - CR0) * NCW;  // compute waves per XCD (210: at most two units per phase)
constexpr int RSN = D / NR;           // outputs per workgroup in a reduce-scatter
constexpr int GS = F / NX;            // GELU slice of an XCD
constexpr int GPS = GS / 64;          // groups per slice
constexpr int NG_PR = F / 64;         // int8 MLP-projection groups
constexpr int HEAD_MAX_ROWS = (V + NCW * GRID - 1) / (NCW * GRID);
constexpr unsigned SPIN_LIMIT = 1u << 21;
static_assert(RSN * NR == D && GS * NX == F && GPS == PR_SLICE_GROUPS && NX == PR_SLICES, "slices");
static_assert(H > NX && H <= 2 * NX, "one or two heads per XCD");

__device__ __forceinline__ int heads_of(int X) { return X + NX < H ? 2 : 1; }

// Exchange area (64-bit words): local [NX][L][FX_LOC_PER_LAYER], global
// [L][FX_GLB_PER_LAYER], placement [GRID].
constexpr int LO_QKV = 0, LO_ATT = 384, LO_X1 = 512, LO_G = 512 + D, LO_X2 = 512 + D + GS;
static_assert(LO_X2 + D == FX_LOC_PER_LAYER, "local layout");
constexpr int GL_O = 0, GL_P = H * D;  // output-projection terms [12][768]; MLP terms [8 or 48][768]
static_assert(GL_P + NG_PR * D == FX_GLB_PER_LAYER, "global layout");
constexpr size_t LOC_WORDS = (size_t)NX * L * FX_LOC_PER_LAYER;
constexpr size_t GLB_WORDS = (size_t)L * FX_GLB_PER_LAYER;
static_assert(LOC_WORDS + GLB_WORDS + GRID + (size_t)GRID * 8 * 16 <= FX_WORDS, "exchange area");

enum { HDR_EPOCH = 0, HDR_DONE = 1, HDR_ERROR = 2 };
enum { ERR_SPIN = 1, ERR_XCC = 2 };

struct FusedArgs {
  Weights w;
  float* cache;
  float* logits;
  u64* fx;           // exchange area
  u64* sinkw;        // [GRID*8][16]: per-wave line for stores of units a wave does not own
  uint32_t* header;
  char* capture;     // int8 test capture or null
  uint64_t* trace;   // timeline test hook or null: [grid][64] timestamps
  uint32_t token;
  int32_t pos;
};

// Timeline test hook.  Compute workgroups: 0 start; 1+4l block l input ready;
// 2+4l attention output received; 3+4l x1 gathered; 4+4l GELU slice gathered;
// 49 head input ready; 50 head rows done; 51 end; block 5 only: 52 LayerNorm 1
// done, 53/54/56/57 QKV/O/FC/MLP units published (wave 1), 55/58 the two
// reduce-scatters done.  Attention workgroups: 1+4l
// q/k/v received; 2+4l attention output published; 3+4l and 4+4l the two
// reduce-scatters done.
__device__ __forceinline__ void stamp(const uint64_t* trace, int slot) {
  if (trace) ((uint64_t*)trace)[blockIdx.x * 64 + slot] = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ u64 ld_sc1(const u64* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_sc1(u64* p, u64 v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// Inside one XCD: a plain 64-bit store reaches the XCD's L2 (the vector L1 writes
// through); a non-temporal load reads it there.
__device__ __forceinline__ void st_loc(u64* p, u64 v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); }
__device__ __forceinline__ u64 ld_loc(const u64* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint32_t ld32(const uint32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ u64 pack(float v, uint32_t e) { return ((u64)e << 32) | __float_as_uint(v); }
__device__ __forceinline__ uint32_t epoch_of(u64 w) { return (uint32_t)(w >> 32); }

// Workgroup barrier that waits only for this wave's LDS traffic, not for its
// outstanding global loads (register prefetches stay in flight across it).
__device__ __forceinline__ void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Order a wave's LDS writes before its later LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

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

// One wave polls n <= 64*PL words, word k at src[idx(k)], until every word has
// epoch E; lane l returns word l + 64j in v[j].
template <int PL, bool LOCAL, class Idx>
__device__ __forceinline__ void poll(const u64* src, int n, Idx idx, uint32_t E, float (&v)[PL], uint32_t* hdr) {
  const int lane = lane_id();
  uint32_t spins = 0;
  while (true) {
    asm volatile("" ::: "memory");
    u64 w[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int k = lane + 64 * j;
      w[j] = k < n ? (LOCAL ? ld_loc(src + idx(k)) : ld_sc1(src + idx(k))) : pack(0.0f, E);
    }
    bool ok = true;
#pragma unroll
    for (int j = 0; j < PL; ++j) ok &= epoch_of(w[j]) == E;
    if (__all(ok) || give_up(spins, hdr)) {
#pragma unroll
      for (int j = 0; j < PL; ++j) v[j] = __uint_as_float((uint32_t)w[j]);
      return;
    }
  }
}

// All-gather inside the XCD: 64*PL words at src into dst (LDS).
template <int PL>
__device__ __forceinline__ void gather(const u64* src, uint32_t E, float* dst, uint32_t* hdr) {
  float v[PL];
  poll<PL, true>(src, 64 * PL, [](int k) { return k; }, E, v, hdr);
#pragma unroll
  for (int j = 0; j < PL; ++j) dst[lane_id() + 64 * j] = v[j];
}

// Reduce-scatter: the workgroup's outputs o = RSN*rank + i (i < RSN) of a sum of
// NT terms stored term-major at terms[t*D + o].  Lanes i < RSN return
// y = 0 + term_0 + ... + term_{NT-1} (fixed order).
template <int NT>
__device__ __forceinline__ float reduce_scatter(const u64* terms, int rank, uint32_t E, float* scratch,
                                                uint32_t* hdr) {
  constexpr int N = NT * RSN, PL = (N + 63) / 64;
  const int lane = lane_id();
  float v[PL];
  poll<PL, false>(terms, N, [&](int k) { return (k / RSN) * D + RSN * rank + k % RSN; }, E, v, hdr);
#pragma unroll
  for (int j = 0; j < PL; ++j)
    if (lane + 64 * j < N) scratch[lane + 64 * j] = v[j];
  wave_lds_sync();
  float y = 0.0f;
  if (lane < RSN) {
#pragma unroll 8
    for (int t = 0; t < NT; ++t) y = y + scratch[t * RSN + lane];
  }
  return y;
}

// ---- per-wave weight registers ----------------------------------------------
// fp32 (float4 slots): QKV rows k=0,1 -> 3k..3k+2; output-projection quad units
// k=0,1 -> 6+k; FC rows k=0,1 -> 8+3k..; MLP row pairs k=0,1 -> 14+3k..16+3k.
// The head uses the six row triples: head slot s at hbase(s) = 0,3,8,11,14,17.
// int8 (int4 slots): QKV rows 0,1; output-projection units 2; FC rows 3,4; MLP
// units 5,6; head slot s = slot s (7 rows in flight).  sc[] is the lane's weight
// scale for its slot.
//
// Every compute wave issues the same sequence of memory instructions on every
// path: units a wave does not own load a valid row in their place and store to a
// sink word, and the last block loads the first head rows into the slots it frees
// (instead of the next block's weights).  So the compiler's wait counts stay exact
// and a wait for one phase's weights never drains the loads behind it.
template <bool Q8>
struct WRegs;
template <>
struct WRegs<false> {
  f4 r[20];
  float b[4];  // bias of QKV rows 0,1, FC rows 0,1
};
template <>
struct WRegs<true> {
  i4 c[7];
  float sc[7];
  float b[4];
};
__device__ __host__ constexpr int hbase(int s) { return s < 2 ? 3 * s : 8 + 3 * (s - 2); }

// QKV row n of XCD X (n < 192 per head): head hh = n/192, part (q,k,v) = n%192/64,
// coordinate n%64.
__device__ __forceinline__ int qkv_row(int X, int n) {
  const int hh = n / 192, part = (n % 192) / 64, d = n % 64;
  return part * D + DH * (X + NX * hh) + d;
}

// Where a wave's units and head rows are; unit indexes are clamped to valid units.
struct Units {
  int X, cw, nh;  // XCD, compute wave of the XCD, heads of the XCD
  int hw, hstride;
  __device__ int head_row(int s) const { return min(hw + s * hstride, V - 1); }
};

__device__ __forceinline__ void ld_row3(f4* dst, const float* row) {
  const int lane = lane_id();
#pragma unroll
  for (int i = 0; i < 3; ++i) dst[i] = __builtin_nontemporal_load((const f4*)(row + 256 * i + 4 * lane));
}

// Block l's QKV row k into its slots, or (head) head slot k.
template <bool Q8, int k>
__device__ __forceinline__ void load_qkv(WRegs<Q8>& R, const Weights& w, int l, const Units& U, bool head) {
  const int r = qkv_row(U.X, min(U.cw + CW * k, 192 * U.nh - 1));
  const int hr = U.head_row(k);
  if constexpr (!Q8) {
    ld_row3(&R.r[hbase(k)], head ? w.wte + (size_t)hr * D : f32_mat(w, l, M_QKV) + (size_t)r * D);
  } else {
    i4 t[1];
    q8_load_row<D>(t, R.sc[k], head ? q8_codes(w, 0, M_HEAD) : q8_codes(w, l, M_QKV),
                   head ? q8_scales(w, 0, M_HEAD) : q8_scales(w, l, M_QKV), head ? hr : r);
    R.c[k] = t[0];
  }
  R.b[k] = small_p(w, l, sp::B_QKV)[r];
}

// Output projection.  fp32: quad unit u (< 192 per head) = outputs 4(u%192)+q of
// head hh = u/192 in quarter q; lane 16q+j holds inputs 4j..4j+3 of the head.
// int8: unit n = 16u + lane/4 (< 768 per head): output n%768 of head n/768; quad
// member s holds codes 16s..16s+15 of the head group.  (fp32 at the last block
// reloads its units; int8 loads head slot 2.)
__device__ __forceinline__ void o_unit_f32(const Units& U, int k, int& u, int& hh, int& i, int& h) {
  u = min(U.cw + CW * k, 192 * U.nh - 1);
  hh = u / 192;
  i = 4 * (u % 192) + lane_id() / 16;
  h = U.X + NX * hh;
}
__device__ __forceinline__ void o_unit_q8(const Units& U, int& n, int& i, int& h) {
  const int u = min(U.cw, 48 * U.nh - 1);
  n = 16 * u + lane_id() / 4;
  i = n % D;
  h = U.X + NX * (n / D);
}
template <bool Q8, int k>
__device__ __forceinline__ void load_o(WRegs<Q8>& R, const Weights& w, int l, const Units& U, bool head) {
  const int lane = lane_id();
  if constexpr (!Q8) {
    int u, hh, i, h;
    o_unit_f32(U, k, u, hh, i, h);
    R.r[6 + k] = __builtin_nontemporal_load(
        (const f4*)(f32_mat(w, l, M_O) + (size_t)i * D + DH * h + 4 * (lane % 16)));
  } else {
    const int hr = U.head_row(2);
    int n, i, h;
    o_unit_q8(U, n, i, h);
    const int8_t* p = head ? q8_codes(w, 0, M_HEAD) + (size_t)hr * D + 16 * min(lane, D / 16 - 1)
                           : q8_codes(w, l, M_O) + (size_t)i * D + DH * h + 16 * (lane % 4);
    const float* sp_ = head ? q8_scales(w, 0, M_HEAD) + (size_t)hr * H + min(lane, H - 1)
                            : q8_scales(w, l, M_O) + (size_t)i * H + h;
    const i4 c = __builtin_nontemporal_load((const i4*)p);
    const float sc = *sp_;
    R.c[2] = (!head || lane < D / 16) ? c : i4{0, 0, 0, 0};
    R.sc[2] = (!head || lane < H) ? sc : 0.0f;
  }
}

// FC row k of the XCD's slice, or head slot 2+k (fp32) / 3+k (int8).
template <bool Q8, int k>
__device__ __forceinline__ void load_fc(WRegs<Q8>& R, const Weights& w, int l, const Units& U, bool head) {
  const int r = GS * U.X + min(U.cw + CW * k, GS - 1);
  if constexpr (!Q8) {
    const int hr = U.head_row(2 + k);
    ld_row3(&R.r[hbase(2 + k)], head ? w.wte + (size_t)hr * D : f32_mat(w, l, M_FC) + (size_t)r * D);
  } else {
    const int hr = U.head_row(3 + k);
    i4 t[1];
    q8_load_row<D>(t, R.sc[3 + k], head ? q8_codes(w, 0, M_HEAD) : q8_codes(w, l, M_FC),
                   head ? q8_scales(w, 0, M_HEAD) : q8_scales(w, l, M_FC), head ? hr : r);
    R.c[3 + k] = t[0];
  }
  R.b[2 + k] = small_p(w, l, sp::B_FC)[r];
}

// MLP projection.  fp32: row pair u (< 384) = rows 2u, 2u+1 over the XCD's slice;
// pass p, quarter q takes group dot kk = 4p+q: row 2u + kk/6, slice group kk%6.
// int8: unit n = 16u + lane/4 (< 6*768): output n/6, group 6X + n%6.  Head
// alternative: fp32 head slot 4+k, int8 head slot 5+k.
template <bool Q8, int k>
__device__ __forceinline__ void load_pr(WRegs<Q8>& R, const Weights& w, int l, const Units& U, bool head) {
  const int lane = lane_id();
  if constexpr (!Q8) {
    const int hr = U.head_row(4 + k);
    const int u = min(U.cw + CW * k, D / 2 - 1);
    const float* W = f32_mat(w, l, M_PR);
    const int q = lane / 16, j = lane % 16;
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const int kk = 4 * p + q, row = 2 * u + kk / GPS, g = GPS * U.X + kk % GPS;
      const float* src = head ? w.wte + (size_t)hr * D + 256 * p + 4 * lane : W + (size_t)row * F + 64 * g + 4 * j;
      R.r[hbase(4 + k) + p] = __builtin_nontemporal_load((const f4*)src);
    }
  } else {
    const int hr = U.head_row(5 + k);
    const int u = min(U.cw + CW * k, GPS * D / 16 - 1);
    const int n = 16 * u + lane / 4, i = n / GPS, g = GPS * U.X + n % GPS;
    const int8_t* p = head ? q8_codes(w, 0, M_HEAD) + (size_t)hr * D + 16 * min(lane, D / 16 - 1)
                           : q8_codes(w, l, M_PR) + (size_t)i * F + 64 * g + 16 * (lane % 4);
    const float* sp_ = head ? q8_scales(w, 0, M_HEAD) + (size_t)hr * H + min(lane, H - 1)
                            : q8_scales(w, l, M_PR) + (size_t)i * NG_PR + g;
    const i4 c = __builtin_nontemporal_load((const i4*)p);
    const float sc = *sp_;
    R.c[5 + k] = (!head || lane < D / 16) ? c : i4{0, 0, 0, 0};
    R.sc[5 + k] = (!head || lane < H) ? sc : 0.0f;
  }
}

template <bool Q8>
constexpr int head_slots() { return Q8 ? 7 : 6; }

// Head row r (clamped to the last row) into head slot s.
template <bool Q8>
__device__ __forceinline__ void load_head(WRegs<Q8>& R, const Weights& w, int s, int r) {
  r = min(r, V - 1);
  if constexpr (!Q8) {
    ld_row3(&R.r[hbase(s)], w.wte + (size_t)r * D);
  } else {
    i4 t[1];
    q8_load_row<D>(t, R.sc[s], q8_codes(w, 0, M_HEAD), q8_scales(w, 0, M_HEAD), r);
    R.c[s] = t[0];
  }
}

// int8 group accumulator of a quad: lanes 4k..4k+3 each hold 16 codes of one group.
__device__ __forceinline__ int quad_acc(const i4 wc, const i4 xc) {
  int p = 0;
  p = __builtin_amdgcn_sdot4(wc.x, xc.x, p, false);
  p = __builtin_amdgcn_sdot4(wc.y, xc.y, p, false);
  p = __builtin_amdgcn_sdot4(wc.z, xc.z, p, false);
  p = __builtin_amdgcn_sdot4(wc.w, xc.w, p, false);
  return quad_sum(p);
}

struct FusedSmem {
  float xs[D];         // block input x, then x1 (all-gathers)
  float xn[D];         // int8 path: LayerNorm output
  float lntmp[D];      // int8 path: LayerNorm scratch
  float att[2 * DH];   // attention output of the XCD's heads
  float xg[GS];        // the XCD's GELU slice
  float rs[NG_PR * RSN];  // reduce-scatter terms
  float lnp[2][4][D];  // LayerNorm parameters by block parity: ln1 gamma, beta, ln2 gamma, beta
  float lnf[2][D];     // final LayerNorm gamma, beta
  int8_t xc[F];        // int8 path: input codes (by input index)
  float xsc[64];       // int8 path: input scales (by group)
  AttnSmem at;         // attention workgroups
};

// Per-workgroup constants.
struct Ctx {
  uint32_t E;  // this launch's epoch
  int X;       // XCD
  int rank;    // rank inside the XCD
  u64* loc;    // this XCD's local words, block 0
  u64* glb;    // global words, block 0
};
__device__ __forceinline__ u64* loc_of(const Ctx& c, int l) { return c.loc + (size_t)l * FX_LOC_PER_LAYER; }
__device__ __forceinline__ u64* glb_of(const Ctx& c, int l) { return c.glb + (size_t)l * FX_GLB_PER_LAYER; }

// 768-vector from global memory into LDS (one wave).
__device__ __forceinline__ void stage_vec(float* dst, const float* src) {
  const int lane = lane_id();
  f4 v[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) v[i] = *(const f4*)(src + 256 * i + 4 * lane);
#pragma unroll
  for (int i = 0; i < 3; ++i) *(f4*)(dst + 256 * i + 4 * lane) = v[i];
}
__device__ __forceinline__ void stage_ln(FusedSmem& S, const Weights& w, int l) {
  float(*p)[D] = S.lnp[l & 1];
  stage_vec(p[0], small_p(w, l, sp::LN1_G));
  stage_vec(p[1], small_p(w, l, sp::LN1_B));
  stage_vec(p[2], small_p(w, l, sp::LN2_G));
  stage_vec(p[3], small_p(w, l, sp::LN2_B));
}

// x = wte[token] + wpe[pos] into LDS; lanes < RSN return element RSN*rank + lane.
__device__ __forceinline__ float embed(const FusedArgs& a, float* xs, int rank) {
  const int lane = lane_id();
#pragma unroll
  for (int j = 0; j < 12; ++j) {
    const int i = lane + 64 * j;
    xs[i] = a.w.wte[(size_t)a.token * D + i] + a.w.wpe[(size_t)a.pos * D + i];
  }
  const int o = RSN * rank + min(lane, RSN - 1);
  return a.w.wte[(size_t)a.token * D + o] + a.w.wpe[(size_t)a.pos * D + o];
}

// The two reduce-scatters of block l (wave 0 of every workgroup).  xr holds the
// residual of this workgroup's outputs (lanes < RSN) and is updated.
template <bool Q8, bool CAP>
__device__ __forceinline__ void rs_o(const FusedArgs& a, FusedSmem& S, const Ctx& c, int l, float& xr) {
  const int lane = lane_id();
  float y = reduce_scatter<H>(glb_of(c, l) + GL_O, c.rank, c.E, S.rs, a.header);
  if (lane < RSN) {
    const int o = RSN * c.rank + lane;
    y = y + small_p(a.w, l, sp::B_O)[o];
    if (CAP && c.X == 0) ((float*)(a.capture + cap_offset(l, M_O) + cap_item(M_O).y))[o] = y;
    xr = xr + y;
    st_loc(loc_of(c, l) + LO_X1 + o, pack(xr, c.E));
  }
}
template <bool Q8, bool CAP>
__device__ __forceinline__ void rs_pr(const FusedArgs& a, FusedSmem& S, const Ctx& c, int l, float& xr) {
  const int lane = lane_id();
  float y = reduce_scatter<Q8 ? NG_PR : NX>(glb_of(c, l) + GL_P, c.rank, c.E, S.rs, a.header);
  if (lane < RSN) {
    const int o = RSN * c.rank + lane;
    y = y + small_p(a.w, l, sp::B_PR)[o];
    if (CAP && c.X == 0) ((float*)(a.capture + cap_offset(l, M_PR) + cap_item(M_PR).y))[o] = y;
    xr = xr + y;
    st_loc(loc_of(c, l) + LO_X2 + o, pack(xr, c.E));
  }
}

// int8: quantize groups g0, g0+gstep, ... (< g1) of src (LDS, indexed from group
// gsrc0) into xc/xsc by input index, one group per compute wave (waves 1..7).
__device__ __forceinline__ void quantize_groups(FusedSmem& S, const float* src, int gsrc0, int g0, int g1, int wave) {
  const int lane = lane_id();
  for (int g = g0 + (wave - 1); g < g1; g += NCW) {
    float s;
    const int q = quant_lane(src[(g - gsrc0) * 64 + lane], s);
    S.xc[g * 64 + lane] = (int8_t)q;
    if (lane == 0) S.xsc[g] = s;
  }
}

// int8 capture of a projection input (fp32 values, codes, scales) for inputs
// [k0, k1) of matrix m at block l; src is indexed from k0.
__device__ __forceinline__ void capture_input(const FusedArgs& a, FusedSmem& S, int l, int m, const float* src, int k0,
                                              int k1, int tid, int nthr) {
  char* base = a.capture + cap_offset(l, m);
  const CapLayout cl = cap_item(m);
  for (int i = k0 + tid; i < k1; i += nthr) {
    ((float*)(base + cl.in))[i] = src[i - k0];
    ((int8_t*)(base + cl.codes))[i] = S.xc[i];
    if (i % 64 == 0) ((float*)(base + cl.xs))[i / 64] = S.xsc[i / 64];
  }
}

// ---- compute workgroups: wave 0 ---------------------------------------------------
template <bool Q8, bool CAP>
__device__ void io_wave(const FusedArgs a, FusedSmem& S, const Ctx c) {
  const int lane = lane_id();
  uint32_t* hdr = a.header;
  // the capture of LayerNorm-output inputs is written by one workgroup, that of the
  // XCD's GELU slice by one workgroup per XCD
  const bool cap0 = CAP && c.X == 0 && c.rank == CR0;
  const bool capx = CAP && c.rank == CR0;
  auto qbar = [&](int l, int m, bool cap) {  // int8: barrier after the compute waves quantized
    if constexpr (Q8) {
      wg_barrier();
      if (cap) {
        if (m == M_PR) capture_input(a, S, l, m, S.xg, GS * c.X, GS * (c.X + 1), lane, 64);
        else capture_input(a, S, l, m, S.xn, 0, D, lane, 64);
      }
    }
  };
  stage_ln(S, a.w, 0);
  stage_vec(S.lnf[0], a.w.small + sp::LNF_G);
  stage_vec(S.lnf[1], a.w.small + sp::LNF_B);
  float xr = embed(a, S.xs, c.rank);  // lanes < RSN: residual of this workgroup's reduce-scatter outputs
  wg_barrier();  // B0: block 0's input and LayerNorm parameters are in LDS
  for (int l = 0; l < L; ++l) {
    const float(*lp)[D] = S.lnp[l & 1];
    u64* loc = loc_of(c, l);
    if (lane == 0) stamp(a.trace, 1 + 4 * l);
    if constexpr (Q8) layernorm_seq(S.xs, lp[0], lp[1], S.xn, S.lntmp);
    if (l == 5 && lane == 0) stamp(a.trace, 52);
    wg_barrier();  // B1: QKV
    qbar(l, M_QKV, cap0);
    // while the XCD's attention runs: next block's LayerNorm parameters
    if (l + 1 < L) stage_ln(S, a.w, l + 1);
    {
      float v[2];
      poll<2, true>(loc + LO_ATT, DH * heads_of(c.X), [](int k) { return k; }, c.E, v, hdr);
      S.att[lane] = v[0];
      S.att[lane + 64] = v[1];
      if (lane == 0) stamp(a.trace, 2 + 4 * l);
    }
    wg_barrier();  // B2: output projection
    qbar(l, M_O, false);
    rs_o<Q8, CAP>(a, S, c, l, xr);
    if (l == 5 && lane == 0) stamp(a.trace, 55);
    gather<12>(loc + LO_X1, c.E, S.xs, hdr);
    if (lane == 0) stamp(a.trace, 3 + 4 * l);
    if constexpr (Q8) layernorm_seq(S.xs, lp[2], lp[3], S.xn, S.lntmp);
    wg_barrier();  // B3: FC
    qbar(l, M_FC, cap0);
    gather<GS / 64>(loc + LO_G, c.E, S.xg, hdr);
    if (lane == 0) stamp(a.trace, 4 + 4 * l);
    wg_barrier();  // B4: MLP projection
    qbar(l, M_PR, capx);
    rs_pr<Q8, CAP>(a, S, c, l, xr);
    if (l == 5 && lane == 0) stamp(a.trace, 58);
    gather<12>(loc + LO_X2, c.E, S.xs, hdr);
  }
  if (lane == 0) stamp(a.trace, 49);
  if constexpr (Q8) layernorm_seq(S.xs, S.lnf[0], S.lnf[1], S.xn, S.lntmp);
  wg_barrier();  // B5: head
  qbar(0, M_HEAD, cap0);
}

// Head rows of wave hw (rows hw + k*hstride): slots were loaded ahead; each slot is
// refilled with the row NS further on as soon as it has been used.  Rows past the
// vocabulary compute on the last row and store to the sink.
template <bool Q8, bool CAP>
__device__ __forceinline__ void head_rows(const FusedArgs a, FusedSmem& S, WRegs<Q8>& R, int hw, int hstride) {
  const int lane = lane_id();
  f4 x[3];
  if constexpr (!Q8) {
    load_frag<3>(x, S.xs);
    layernorm_frag(x, S.lnf[0], S.lnf[1]);
  }
  constexpr int NS = head_slots<Q8>();
#pragma unroll
  for (int k = 0; k < HEAD_MAX_ROWS; ++k) {
    // keep the loads in slot order: at most NS rows in flight per wave
    __builtin_amdgcn_sched_barrier(0);
    const int r = hw + k * hstride;
    const int s = k % NS;
    float y;
    if constexpr (!Q8) {
      y = dot_frag<3>(*reinterpret_cast<f4(*)[3]>(&R.r[hbase(s)]), x);
    } else {
      int32_t* ca = CAP && r < V ? (int32_t*)(a.capture + cap_offset(0, M_HEAD) + cap_item(M_HEAD).acc) + (size_t)r * 12
                                 : nullptr;
      y = q8_dot<D>(*reinterpret_cast<i4(*)[1]>(&R.c[s]), R.sc[s], S.xc, S.xsc, ca);
      if (CAP && r < V && lane == 0) ((float*)(a.capture + cap_offset(0, M_HEAD) + cap_item(M_HEAD).y))[r] = y;
    }
    *(r < V ? a.logits + r : (float*)(a.sinkw + ((size_t)blockIdx.x * 8 + (threadIdx.x >> 6)) * 16 + 8)) = y;
    load_head<Q8>(R, a.w, s, r + NS * hstride);
  }
}

// ---- compute workgroups: waves 1..7 -----------------------------------------------
template <bool Q8, bool CAP>
__device__ void compute_waves(const FusedArgs a, FusedSmem& S, const Ctx c) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int X = c.X;
  Units U;
  U.X = X;
  U.cw = (wave - 1) * (NR - CR0) + (c.rank - CR0);  // compute wave of the XCD
  U.nh = heads_of(X);
  U.hw = (wave - 1) * GRID + (int)blockIdx.x;  // first head row
  U.hstride = NCW * GRID;
  const int cw = U.cw, nh = U.nh;
  const uint32_t E = c.E;
  // this wave's own sink line (stores of different waves never meet)
  u64* sinkw = a.sinkw + ((size_t)blockIdx.x * 8 + wave) * 16;
  float* sinkf = (float*)(sinkw + 8);
  auto qsync = [&]() {
    if constexpr (Q8) wg_barrier();
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;

  WRegs<Q8> R;
  load_qkv<Q8, 0>(R, a.w, 0, U, false);
  load_qkv<Q8, 1>(R, a.w, 0, U, false);
  load_o<Q8, 0>(R, a.w, 0, U, false);
  if constexpr (!Q8) load_o<Q8, 1>(R, a.w, 0, U, false);
  load_fc<Q8, 0>(R, a.w, 0, U, false);
  load_fc<Q8, 1>(R, a.w, 0, U, false);
  load_pr<Q8, 0>(R, a.w, 0, U, false);
  load_pr<Q8, 1>(R, a.w, 0, U, false);
  wg_barrier();  // B0

  for (int l = 0; l < L; ++l) {
    u64* loc = loc_of(c, l);
    u64* glb = glb_of(c, l);
    const bool last = l + 1 == L;
    const int ln = last ? l : l + 1;  // block whose weights are loaded next (head rows after the last)
    // ---- QKV rows; k/v rows also go to the cache
    wg_barrier();  // B1
    if constexpr (Q8) {
      quantize_groups(S, S.xn, 0, 0, D / 64, wave);
      qsync();
    }
    {
      f4 x[3];
      if constexpr (!Q8) {
        load_frag<3>(x, S.xs);
        layernorm_frag(x, S.lnp[l & 1][0], S.lnp[l & 1][1]);
      }
      auto row = [&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const int n = cw + CW * k;
        const bool own = n < 192 * nh;
        const int r = qkv_row(X, own ? n : 0);
        float y;
        if constexpr (!Q8) {
          y = dot_frag<3>(*reinterpret_cast<f4(*)[3]>(&R.r[hbase(k)]), x);
        } else {
          int32_t* ca = CAP && own ? (int32_t*)(a.capture + cap_offset(l, M_QKV) + cap_item(M_QKV).acc) + (size_t)r * 12
                                   : nullptr;
          y = q8_dot<D>(*reinterpret_cast<i4(*)[1]>(&R.c[k]), R.sc[k], S.xc, S.xsc, ca);
        }
        y = y + R.b[k];
        st_loc(own ? loc + LO_QKV + n : sinkw, pack(y, E));
        *(own && r >= D ? a.cache + ((size_t)a.pos * L + l) * KV_ROW + (r - D) : sinkf) = y;
        if (CAP && own && lane == 0) ((float*)(a.capture + cap_offset(l, M_QKV) + cap_item(M_QKV).y))[r] = y;
        load_qkv<Q8, k>(R, a.w, ln, U, last);
      };
      row(K0{});
      row(K1{});
    }
    if (l == 5 && wave == 1 && lane == 0) stamp(a.trace, 53);
    // ---- output projection: one term per (head, output)
    wg_barrier();  // B2
    if constexpr (Q8) {
      // the XCD's head groups: wave 1 quantizes head X, wave 2 head X + 8
      if (wave - 1 < nh) {
        const int hh = wave - 1, g = X + NX * hh;
        float s;
        const int q = quant_lane(S.att[DH * hh + lane], s);
        S.xc[64 * g + lane] = (int8_t)q;
        if (lane == 0) S.xsc[g] = s;
      }
      qsync();
    }
    if constexpr (!Q8) {
      auto unit = [&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const bool own = cw + CW * k < 192 * nh;
        int u, hh, i, h;
        o_unit_f32(U, k, u, hh, i, h);
        const f4 xv = *(const f4*)(S.att + DH * hh + 4 * (lane % 16));
        const float p = dot_q16(R.r[6 + k], xv);
        st_sc1(own ? glb + GL_O + (size_t)h * D + i : sinkw, pack(p, E));
        load_o<Q8, k>(R, a.w, ln, U, last);
      };
      unit(K0{});
      unit(K1{});
    } else {
      const bool own = cw < 48 * nh;
      int n, i, h;
      o_unit_q8(U, n, i, h);
      const i4 xv = *(const i4*)(S.xc + DH * h + 16 * (lane % 4));
      const int acc = quad_acc(R.c[2], xv);
      const float t = ((float)acc * R.sc[2]) * S.xsc[h];
      st_sc1(own ? glb + GL_O + (size_t)h * D + i : sinkw, pack(t, E));
      if (CAP && own && lane % 4 == 0)
        ((int32_t*)(a.capture + cap_offset(l, M_O) + cap_item(M_O).acc))[(size_t)i * H + h] = acc;
      load_o<Q8, 0>(R, a.w, ln, U, last);
    }
    if (l == 5 && wave == 1 && lane == 0) stamp(a.trace, 54);
    // ---- FC rows and GELU
    wg_barrier();  // B3
    if constexpr (Q8) {
      quantize_groups(S, S.xn, 0, 0, D / 64, wave);
      qsync();
    }
    {
      f4 x[3];
      if constexpr (!Q8) {
        load_frag<3>(x, S.xs);
        layernorm_frag(x, S.lnp[l & 1][2], S.lnp[l & 1][3]);
      }
      auto row = [&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const int n = cw + CW * k;
        const bool own = n < GS;
        const int r = GS * X + (own ? n : 0);
        float y;
        if constexpr (!Q8) {
          y = dot_frag<3>(*reinterpret_cast<f4(*)[3]>(&R.r[hbase(2 + k)]), x);
        } else {
          int32_t* ca = CAP && own ? (int32_t*)(a.capture + cap_offset(l, M_FC) + cap_item(M_FC).acc) + (size_t)r * 12
                                   : nullptr;
          y = q8_dot<D>(*reinterpret_cast<i4(*)[1]>(&R.c[3 + k]), R.sc[3 + k], S.xc, S.xsc, ca);
        }
        y = y + R.b[2 + k];
        st_loc(own ? loc + LO_G + n : sinkw, pack(gelu_tanh(y), E));
        if (CAP && own && lane == 0) ((float*)(a.capture + cap_offset(l, M_FC) + cap_item(M_FC).y))[r] = y;
        load_fc<Q8, k>(R, a.w, ln, U, last);
      };
      row(K0{});
      row(K1{});
    }
    if (l == 5 && wave == 1 && lane == 0) stamp(a.trace, 56);
    // ---- MLP projection: fp32 one partial per (slice, output), int8 one term per
    // (group, output)
    wg_barrier();  // B4
    if constexpr (Q8) {
      quantize_groups(S, S.xg, GPS * X, GPS * X, GPS * (X + 1), wave);
      qsync();
    }
    if constexpr (!Q8) {
      auto unit = [&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const int u0 = cw + CW * k;
        const bool own = u0 < D / 2;
        const int u = own ? u0 : 0;
        const int q = lane / 16, j = lane % 16;
        float qv[3];
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          const int kk = 4 * p + q;
          const f4 xv = *(const f4*)(S.xg + 64 * (kk % GPS) + 4 * j);
          qv[p] = dot_q16(R.r[hbase(4 + k) + p], xv);
        }
        auto val = [&](int kk) { return lane_val(qv[kk / 4], 16 * (kk % 4)); };
        float p0 = val(0), p1 = val(GPS);
#pragma unroll
        for (int kk = 1; kk < GPS; ++kk) {
          p0 = p0 + val(kk);
          p1 = p1 + val(GPS + kk);
        }
        // lanes 0..31 store row 2u, lanes 32..63 row 2u+1
        const int half = lane >> 5;
        st_sc1(own ? glb + GL_P + (size_t)X * D + 2 * u + half : sinkw, pack(half ? p1 : p0, E));
        load_pr<Q8, k>(R, a.w, ln, U, last);
      };
      unit(K0{});
      unit(K1{});
    } else {
      auto unit = [&](auto kc) {
        constexpr int k = decltype(kc)::value;
        const int u0 = cw + CW * k;
        const bool own = u0 < GPS * D / 16;
        const int n = 16 * (own ? u0 : 0) + lane / 4, i = n / GPS, g = GPS * X + n % GPS;
        const i4 xv = *(const i4*)(S.xc + 64 * g + 16 * (lane % 4));
        const int acc = quad_acc(R.c[5 + k], xv);
        const float t = ((float)acc * R.sc[5 + k]) * S.xsc[g];
        st_sc1(own ? glb + GL_P + (size_t)g * D + i : sinkw, pack(t, E));
        if (CAP && own && lane % 4 == 0)
          ((int32_t*)(a.capture + cap_offset(l, M_PR) + cap_item(M_PR).acc))[(size_t)i * NG_PR + g] = acc;
        load_pr<Q8, k>(R, a.w, ln, U, last);
      };
      unit(K0{});
      unit(K1{});
    }
    if (l == 5 && wave == 1 && lane == 0) stamp(a.trace, 57);
  }
  // the head: its first rows were loaded during the last block
  wg_barrier();  // B5
  if constexpr (Q8) {
    quantize_groups(S, S.xn, 0, 0, D / 64, wave);
    qsync();
  }
  head_rows<Q8, CAP>(a, S, R, U.hw, U.hstride);
  if (wave == 1 && lane == 0) stamp(a.trace, 50);
}

// ---- attention workgroups (ranks 0 and 1): head X + 8*rank when it exists ----------
template <bool Q8, bool CAP>
__device__ void attention_wg(const FusedArgs a, FusedSmem& S, const Ctx c) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const bool has_head = c.rank < heads_of(c.X);
  const int h = c.X + NX * c.rank, pos = a.pos;
  uint32_t* hdr = a.header;
  AttnSmem& sm = S.at;
  const int hw = (wave - 1) * GRID + (int)blockIdx.x;  // head rows of waves 1..7
  const int hstride = NCW * GRID;
  float xr = 0.0f;
  if (wave == 0) {
    stage_vec(S.lnf[0], a.w.small + sp::LNF_G);
    stage_vec(S.lnf[1], a.w.small + sp::LNF_B);
    xr = embed(a, S.xs, c.rank);
  }
  for (int l = 0; l < L; ++l) {
    u64* loc = loc_of(c, l);
    if (has_head) {
      const float* cl = a.cache + (size_t)l * KV_ROW + h * DH;
      auto kv = [&](int j) { return cl + (size_t)j * CACHE_POS; };
      attn_stage_rows(sm, kv, 0, pos, 64, FT - 64);
      if (wave == 0) {
        float v[3];
        poll<3, true>(loc + LO_QKV + 192 * c.rank, 192, [](int k) { return k; }, c.E, v, hdr);
        if (lane == 0) stamp(a.trace, 1 + 4 * l);
        sm.q[lane] = v[0];
        sm.k[pos][lane] = v[1];
        sm.v[pos][lane] = v[2];
      }
      __syncthreads();
      const float o = Q8 ? attn_compute_seq(sm, pos + 1) : attn_compute(sm, pos + 1, FT / 64);
      if (wave == 0) {
        st_loc(loc + LO_ATT + DH * c.rank + lane, pack(o, c.E));
        if (lane == 0) stamp(a.trace, 2 + 4 * l);
        if (CAP) {
          float s;
          const int q = quant_lane(o, s);
          char* base = a.capture + cap_offset(l, M_O);
          const CapLayout cl2 = cap_item(M_O);
          ((float*)(base + cl2.in))[DH * h + lane] = o;
          ((int8_t*)(base + cl2.codes))[DH * h + lane] = (int8_t)q;
          if (lane == 0) ((float*)(base + cl2.xs))[h] = s;
        }
      }
      __syncthreads();  // the LDS rows are free for the next block
    }
    if (wave == 0) {
      rs_o<Q8, CAP>(a, S, c, l, xr);
      if (lane == 0) stamp(a.trace, 3 + 4 * l);
      rs_pr<Q8, CAP>(a, S, c, l, xr);
      if (lane == 0) stamp(a.trace, 4 + 4 * l);
    }
  }
  // the tied head: these workgroups take head rows too
  WRegs<Q8> R;
  if (wave >= 1) {
#pragma unroll
    for (int s = 0; s < head_slots<Q8>(); ++s) load_head<Q8>(R, a.w, s, hw + s * hstride);
  }
  if (wave == 0) {
    gather<12>(loc_of(c, L - 1) + LO_X2, c.E, S.xs, hdr);
    if constexpr (Q8) layernorm_seq(S.xs, S.lnf[0], S.lnf[1], S.xn, S.lntmp);
  }
  wg_barrier();
  if (wave >= 1) {
    if constexpr (Q8) quantize_groups(S, S.xn, 0, 0, D / 64, wave);
  }
  if constexpr (Q8) wg_barrier();
  if (wave >= 1) head_rows<Q8, CAP>(a, S, R, hw, hstride);
}

template <bool Q8, bool CAP>
__global__ __launch_bounds__(FT, 1) void k_fused(const FusedArgs a) {
  extern __shared__ __align__(16) char smem_raw[];
  FusedSmem& S = *(FusedSmem*)smem_raw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint32_t* hdr = a.header;
  if (threadIdx.x == 0) stamp(a.trace, 0);
  Ctx c;
  c.E = ld32(&hdr[HDR_EPOCH]) + 1u;
  c.X = (int)xcc_id();
  c.rank = (int)blockIdx.x / NX;
  if (c.X >= NX) {
    if (threadIdx.x == 0) set_error(hdr, ERR_XCC);
    c.X = 0;
  }
  c.loc = a.fx + (size_t)c.X * L * FX_LOC_PER_LAYER;
  c.glb = a.fx + LOC_WORDS;
  if (c.rank < CR0) attention_wg<Q8, CAP>(a, S, c);
  else if (wave == 0) io_wave<Q8, CAP>(a, S, c);
  else compute_waves<Q8, CAP>(a, S, c);

  __syncthreads();
  if (threadIdx.x == 0) {
    stamp(a.trace, 51);
    u64* place = a.fx + LOC_WORDS + GLB_WORDS;
    st_sc1(place + blockIdx.x, ((u64)c.E << 32) | (uint32_t)c.X);
    const uint32_t done = atomicAdd(&hdr[HDR_DONE], 1u);
    if (done == (uint32_t)GRID - 1) {
      // placement check: XCD(b) - b must be one constant mod NX for the rank/XCD
      // split above to hold (the waits would have given up otherwise)
      int off = -1;
      bool bad = false;
      uint32_t spins = 0;  // one bound for the whole check
      for (int b = 0; b < GRID; ++b) {
        u64 w;
        do {
          w = ld_sc1(place + b);
        } while (epoch_of(w) != c.E && ++spins < SPIN_LIMIT);
        const int o = ((int)(uint32_t)w - b % NX + NX) % NX;
        if (off < 0) off = o;
        bad |= o != off || epoch_of(w) != c.E;
      }
      if (bad) set_error(hdr, ERR_XCC);
      hdr[HDR_DONE] = 0;
      __hip_atomic_store(&hdr[HDR_EPOCH], c.E, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---- host side ---------------------------------------------------------------

struct FusedConfig {
  int ok;  // 1 usable, 0 not yet probed, -1 unusable (fall back to per-phase kernels)
};
static FusedConfig g_cfg[3][64];
uint64_t* g_fused_trace = nullptr;  // timeline test hook
int g_fused_plain_launch = 1;       // 1: ordinary launch (default), 0: cooperative launch

template <bool Q8, bool CAP>
static hipError_t fused_config(FusedConfig& c) {
  if (c.ok) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev))) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev))) return e;
  const size_t lds = sizeof(FusedSmem);
  if ((e = hipFuncSetAttribute((const void*)k_fused<Q8, CAP>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)))
    return e;
  int per_cu = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_fused<Q8, CAP>, FT, lds))) return e;
  // One workgroup per compute unit, 32 per XCD: the grid is the whole chip.
  c.ok = (cus == GRID && per_cu >= 1) ? 1 : -1;
  return hipSuccess;
}

template <bool Q8, bool CAP>
static hipError_t launch_fused_t(const Weights& w, const Work& k, uint32_t token, int32_t pos, float* cache,
                                 float* logits, char* capture, hipStream_t s, bool* used) {
  *used = false;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e) return e;
  FusedConfig& c = g_cfg[Q8 ? (CAP ? 2 : 1) : 0][dev & 63];
  if ((e = fused_config<Q8, CAP>(c))) return e;
  if (c.ok != 1) return hipSuccess;
  FusedArgs a{};
  a.w = w;
  a.cache = cache;
  a.logits = logits;
  a.fx = k.ll;
  a.sinkw = k.ll + LOC_WORDS + GLB_WORDS + GRID;
  a.header = k.header;
  a.capture = capture;
  a.trace = g_fused_trace;
  a.token = token;
  a.pos = pos;
  void* args[] = {&a};
  if (g_fused_plain_launch)
    e = hipLaunchKernel((const void*)k_fused<Q8, CAP>, dim3(GRID), dim3(FT), args, sizeof(FusedSmem), s);
  else
    e = hipLaunchCooperativeKernel((const void*)k_fused<Q8, CAP>, dim3(GRID), dim3(FT), args, sizeof(FusedSmem), s);
  if (e == hipSuccess) *used = true;
  return e;
}

hipError_t launch_fused(bool q8, const Weights& w, const Work& k, uint32_t token, int32_t pos, float* cache,
                        float* logits, char* capture, hipStream_t s, bool* used) {
  if (!q8) return launch_fused_t<false, false>(w, k, token, pos, cache, logits, nullptr, s, used);
  if (capture) return launch_fused_t<true, true>(w, k, token, pos, cache, logits, capture, s, used);
  return launch_fused_t<true, false>(w, k, token, pos, cache, logits, nullptr, s, used);
}

}  // namespace g2
