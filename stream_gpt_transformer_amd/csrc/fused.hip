// Fused single-launch decode step (batch 1): one token through the 12 blocks and
// the tied head (LeanExe GPT-2 README, cachedStep paragraph) in one launch of one
// 512-thread workgroup per compute unit.
//
// Why one launch: a step is a chain of ~60 dependent phases over ~495 MB (fp32) or
// ~137 MB (int8) of weights; a kernel launch per phase costs ~1.7-2.5 us on MI355X,
// more than most phases' own HBM time.
//
// Why two sets of compute units: an exchange between workgroups is a store and a
// poll.  On MI355X a poll from a compute unit that also has HBM loads in flight
// queues behind them (an XCD-local exchange goes from ~0.65 us to ~2.2 us), while
// streaming on other compute units of the same XCD does not slow it.  So the 32
// compute units of each XCD form two sets that alternate by block: set s = rank & 1
// computes blocks s, s+2, ..., and while it computes block l (polls, dot products,
// publishes: no HBM traffic but the key/value row of the new token) the other set
// loads the weights of block l+1 into its registers (and the head's key/value rows
// into LDS).  A unit loads the weights of its next block only after its last
// exchange of the current one.
//
// Placement (Megatron-style over the XCDs, inside each set): workgroup b runs on
// XCD X = b % 8 (the dispatcher deals workgroups round-robin over the XCDs; every
// launch checks it) with rank b / 8; set rank q = rank / 2.  XCD X owns heads X and
// X + 8 (when below 12), FC rows 384X..384X+383 and the matching 384-input slice of
// the MLP projection.  In each set, units q < (heads of X) are head units: the
// attention of head X + 8q with its keys/values in LDS and that head's
// output-projection terms (weights in registers); the others are regular units:
// QKV rows of the XCD's heads, FC rows of the slice and the slice's MLP-projection
// partials (weights in registers of waves 1..7).  Every unit of the set owns 48
// outputs of the two reductions over XCDs (reduce-scatters through device memory).
// Per block: x (all-gather in the XCD) -> LayerNorm, QKV rows -> head unit (XCD
// local) -> attention, output-projection terms (global) -> reduce-scatter x1 ->
// all-gather x1 -> LayerNorm, FC rows, GELU -> all-gather of the GELU slice -> MLP
// partials (global) -> reduce-scatter by the other set, which computes the next
// block: two exchanges across XCDs and four inside one per block.
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

constexpr int FT = 512;                  // threads per workgroup
constexpr int NWV = FT / 64;             // waves per workgroup
constexpr int NX = FX_NXCC;              // XCDs
constexpr int NR = 32;                   // workgroups per XCD
constexpr int GRID = NX * NR;            // 256 = compute units of an MI355X
constexpr int NQ = NR / 2;               // units of one set in one XCD
constexpr int RSN = D / NQ;              // reduce-scatter outputs per unit (48)
constexpr int GS = F / NX;               // FC slice of an XCD (384)
constexpr int GPS = GS / 64;             // groups per slice (6)
constexpr int NG_PR = F / 64;            // int8 MLP-projection groups (48)
constexpr int NCW = NWV - 1;             // compute waves of a regular unit (waves 1..7)
constexpr int UPW = 4;                   // units per compute wave per phase
#ifndef FUSED_MLP_TRED
#define FUSED_MLP_TRED 1
#endif
#ifndef FUSED_TRED
#define FUSED_TRED 1
#endif
#ifndef FUSED_NHS_F32
#define FUSED_NHS_F32 16
#endif
template <bool Q8>
constexpr int nhs() { return Q8 ? 12 : FUSED_NHS_F32; }  // head-row slots per wave
constexpr int F32_SLOTS = 3 * FUSED_NHS_F32 > 24 ? 3 * FUSED_NHS_F32 : 24;  // f4 slots of an fp32 wave
// Head rows: the 1,024 waves of each set take rows first + 1024 k, k < n.  Set 0 is
// idle during block 11, so its waves load their first slots while that block runs;
// set 1's only after it.  Set 0 therefore takes more rows per wave (HEAD_N0) than
// set 1 (HEAD_TOTAL - HEAD_N0), so both have about as many rows left to stream when
// the head starts.
constexpr int HEAD_SET_WAVES = NWV * GRID / 2;
constexpr int HEAD_TOTAL = (V + HEAD_SET_WAVES - 1) / HEAD_SET_WAVES;  // rows per set-0 + set-1 wave pair (50)
#ifndef FUSED_HEAD_N0_F32
#define FUSED_HEAD_N0_F32 31
#endif
#ifndef FUSED_HEAD_N0_Q8
#define FUSED_HEAD_N0_Q8 31
#endif
template <bool Q8>
constexpr int head_n0() { return Q8 ? FUSED_HEAD_N0_Q8 : FUSED_HEAD_N0_F32; }
template <bool Q8>
constexpr int head_nmax() { return head_n0<Q8>() > HEAD_TOTAL - head_n0<Q8>() ? head_n0<Q8>() : HEAD_TOTAL - head_n0<Q8>(); }
struct HeadRows {
  int first, n;  // rows first + HEAD_SET_WAVES * k, k < n
};
// Where every lane of a group holds the same value, every lane stores it (one wave
// instruction, the same address in each lane of the group): masking all but one lane
// per group measured slower.
// Output projection of a head unit: 768 outputs x 64 inputs as 1536 half dots of
// 32 inputs, three per thread.
constexpr int O_HALF_PER_THREAD = 2 * D / FT;
static_assert(O_HALF_PER_THREAD * FT == 2 * D, "half dots per thread");
constexpr unsigned SPIN_LIMIT = 1u << 21;
static_assert(RSN * NQ == D && GS * NX == F && GPS == PR_SLICE_GROUPS && NX == PR_SLICES, "slices");
static_assert(H > NX && H <= 2 * NX, "one or two heads per XCD");
// compute waves of a set in one XCD: 7 * (16 - heads) >= 98
static_assert(UPW * NCW * (NQ - 2) >= 2 * 192 && UPW * NCW * (NQ - 2) >= GS && UPW * NCW * (NQ - 2) >= D / 2 &&
                  UPW * NCW * (NQ - 2) >= GPS * D / 16,
              "units per phase");
static_assert(HEAD_TOTAL - head_n0<true>() >= nhs<true>() && head_n0<true>() >= nhs<true>() &&
                  HEAD_TOTAL - head_n0<false>() >= nhs<false>() && head_n0<false>() >= nhs<false>(),
              "head ring");

__device__ __forceinline__ int heads_of(int X) { return X + NX < H ? 2 : 1; }

// Exchange area (64-bit words): local [NX][L][FX_LOC_PER_LAYER], global
// [L][FX_GLB_PER_LAYER], placement [GRID], sink lines [GRID*8][16].
constexpr int LO_QKV = 0, LO_X1 = 384, LO_G = LO_X1 + D, LO_X2 = LO_G + GS;
static_assert(LO_X2 + D <= FX_LOC_PER_LAYER, "local layout");
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
  int32_t* status_out;  // with clear_error: receives the launch's error word (may be null)
  uint32_t token;
  int32_t pos;
  uint32_t clear_error;  // 1: the last workgroup reports the error word and clears it
};

// Timeline test hook (100 MHz wall clock), per workgroup: 0 start; for block l
// computed by the workgroup's set, 1+4l block input ready (head units: after their
// reduce-scatter), 2+4l QKV rows published (regular, wave 1) / attention output
// ready (head units), 3+4l x1 ready (after the all-gather; head units: their
// reduce-scatter), 4+4l GELU slice gathered; 49 head input ready; 50 head rows
// done; 51 end.
__device__ __forceinline__ void stamp(const uint64_t* trace, int slot) {
  if (trace) ((uint64_t*)trace)[blockIdx.x * 64 + slot] = __builtin_amdgcn_s_memrealtime();
}
// Head phase (wave 1): 55 head LayerNorm done (rows start), 57 the preloaded rows used.
// Detail stamps 52..63 inside block 6 (set 0): regular wave 0: 52 the MLP terms'
// reduce-scatter begins (fp32: its x1 share read; int8: its share of the terms
// polled into LDS), 53 after the workgroup barrier, 54 x published, 56 x1
// published; regular wave 1: 59 after the QKV barrier, 60 LayerNorm done, 62 MLP
// phase start, 63 MLP partials published; head wave 0: 52 its reduce-scatter
// begins, 54 q/k/v received, 56 output-projection terms published.
constexpr int DETAIL_L = 6;
__device__ __forceinline__ void dstamp(const uint64_t* trace, int l, int slot) {
  if (l == DETAIL_L && lane_id() == 0) stamp(trace, slot);
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
// vmcnt(0): every global access this wave issued, its stores included, has completed.
__device__ __forceinline__ void wave_vmem_sync() { __builtin_amdgcn_s_waitcnt(0x0f70); }

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

// All-gather of a 768-vector inside the XCD straight into the lane-fragment layout
// (lane l: elements 256i + 4l .. 256i + 4l + 3, i < 3), the layout load_frag reads
// from LDS, without the pass through LDS.
__device__ __forceinline__ void gather_frag(const u64* src, uint32_t E, f4 (&x)[3], uint32_t* hdr) {
  float v[12];
  poll<12, true>(src, 768, [](int k) {
    const int j = k >> 6;
    return 256 * (j >> 2) + 4 * (k & 63) + (j & 3);
  }, E, v, hdr);
#pragma unroll
  for (int i = 0; i < 3; ++i) x[i] = f4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
}

// Reduce-scatter: the unit's outputs o = RSN*q + i (i < RSN) of a sum of NT terms
// stored term-major at terms[t*D + o], read by one wave with lane i holding the NT
// terms of output RSN*q + i (lanes >= RSN read lane RSN-1's words).  Lanes i < RSN
// return y = 0 + term_0 + ... + term_{NT-1} (fixed order).
template <int NT>
__device__ __forceinline__ float rs_lanes(const u64* terms, int q, uint32_t E, uint32_t* hdr) {
  float v[NT];
  poll<NT, false>(terms, 64 * NT, [&](int k) { return (k >> 6) * D + RSN * q + min(k & 63, RSN - 1); }, E, v, hdr);
  float y = 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t) y = y + v[t];
  return y;
}

// Cooperative poll of a reduce-scatter's NT*RSN terms (NT terms of the unit's RSN
// outputs, term-major at terms[t*D + o]): wave w polls its share into
// scratch[t*RSN + i]; after a workgroup barrier rs_sum adds them.
template <int NT>
__device__ __forceinline__ void rs_poll_part(const u64* terms, int q, uint32_t E, float* scratch, uint32_t* hdr,
                                             int wave) {
  constexpr int N = NT * RSN, PER = (N + NWV - 1) / NWV, PL = (PER + 63) / 64;
  const int lane = lane_id();
  const int k0 = wave * PER, n = min(PER, N - k0);
  float v[PL];
  poll<PL, false>(terms, n, [&](int k) { k += k0; return (k / RSN) * D + RSN * q + k % RSN; }, E, v, hdr);
#pragma unroll
  for (int j = 0; j < PL; ++j)
    if (lane + 64 * j < n) scratch[k0 + lane + 64 * j] = v[j];
}
template <int NT>
__device__ __forceinline__ float rs_sum(const float* scratch) {
  const int lane = lane_id();
  float y = 0.0f;
  if (lane < RSN) {
    // every term is read before the ordered adds, so the chain pays one LDS latency
    float v[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) v[t] = scratch[t * RSN + lane];
#pragma unroll
    for (int t = 0; t < NT; ++t) y = y + v[t];
  }
  return y;
}

// ---- per-wave weight registers ----------------------------------------------
// Regular units, fp32 (float4 slots): QKV rows k < 4 -> 3k..3k+2; FC rows k < 4 ->
// 12+3k..; the MLP row pairs are in LDS (PrLds).  Head units: output-projection
// half dot k < 3 -> slots 8k..8k+7.  Head rows (after the last block): slot triple
// s -> 3s.
// int8 (int4 slots): QKV rows 0..3, FC rows 4..7, MLP units 8..11; head units:
// output-projection half dot k -> slots 2k, 2k+1 and scale sc[k]; head rows: slot s.  sc[] is the lane's weight scale
// for its slot.
// binary16 weights (H16, the block matrices and the head; the embedding rows stay
// fp32): the fp32 slot numbering with four halves per slot, widened to fp32 where
// they are used, so the values and the order of operations are those of the fp32
// step on the same (binary16-representable) weights.
//
// Units a wave does not own load a valid row in their place and store to a sink
// word, so every wave of a role issues the same memory-instruction stream and the
// compiler's wait counts stay exact.
template <bool Q8, bool H16 = false>
struct WRegs;
template <>
struct WRegs<false, false> {
  f4 r[F32_SLOTS];
  float b[8];  // bias of QKV rows 0..3, FC rows 0..3
};
template <>
struct WRegs<false, true> {
  h4 r[F32_SLOTS];
  float b[8];
};
template <>
struct WRegs<true, false> {
  i4 c[12];
  float sc[12];
  float b[8];
};
// fp32 weight slot s (H16: widened)
template <bool H16>
__device__ __forceinline__ f4 wslot(const WRegs<false, H16>& R, int s) {
  if constexpr (H16) return widen(R.r[s]);
  else return R.r[s];
}
// dot_frag of the 768-weight row in slots s..s+2 with x
template <bool H16>
__device__ __forceinline__ float dot_slots(WRegs<false, H16>& R, int s, const f4 (&x)[3]) {
  if constexpr (H16) {
    const f4 wv[3] = {widen(R.r[s]), widen(R.r[s + 1]), widen(R.r[s + 2])};
    return dot_frag<3>(wv, x);
  } else {
    return dot_frag<3>(*reinterpret_cast<f4(*)[3]>(&R.r[s]), x);
  }
}

// dot_slots' lane partial (before the wave sum)
template <bool H16>
__device__ __forceinline__ float dot_slots_lane(WRegs<false, H16>& R, int s, const f4 (&x)[3]) {
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const f4 w = wslot(R, s + i);
    acc = fmaf(w.x, x[i].x, acc);
    acc = fmaf(w.y, x[i].y, acc);
    acc = fmaf(w.z, x[i].z, acc);
    acc = fmaf(w.w, x[i].w, acc);
  }
  return acc;
}
// A compute wave's UPW rows of one phase (slots and biases B0..B0+UPW-1) reduced
// together (wave_treduce: wave_sum's bits for each row): lane t returns row
// k = treduce_out<UPW>(t % 16) plus its bias, and k.
template <int B0, bool H16>
__device__ __forceinline__ float rows_treduce(WRegs<false, H16>& R, const f4 (&x)[3], int& k) {
  float lp[UPW];
#pragma unroll
  for (int j = 0; j < UPW; ++j) lp[j] = dot_slots_lane(R, 3 * (B0 + j), x);
  k = treduce_out<UPW>(lane_id() & 15);
  // the lane's bias by selects on register values (a select between elements of R.b
  // would be folded into an indexed load, which puts R in scratch memory)
  float bb[UPW];
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    bb[j] = R.b[B0 + j];
    asm volatile("" : "+v"(bb[j]));
  }
  float b = bb[0];
#pragma unroll
  for (int j = 1; j < UPW; ++j) b = k == j ? bb[j] : b;
  return wave_treduce<UPW>(lp) + b;
}

// QKV row n of XCD X (n < 192 per head): head hh = n/192, part (q,k,v) = n%192/64,
// coordinate n%64.
__device__ __forceinline__ int qkv_row(int X, int n) {
  const int hh = n / 192, part = (n % 192) / 64, d = n % 64;
  return part * D + DH * (X + NX * hh) + d;
}

// Where a regular compute wave's units are; unit indexes are clamped to valid units.
struct Units {
  int X, cw, cwn, nh;  // XCD, compute wave of the XCD's set, compute waves of the set, heads of the XCD
  __device__ int qkv(int k) const { return cw + cwn * k; }
};

__device__ __forceinline__ void ld_row3(f4* dst, const float* row) {
  const int lane = lane_id_fresh();
#pragma unroll
  for (int i = 0; i < 3; ++i) dst[i] = __builtin_nontemporal_load((const f4*)(row + 256 * i + 4 * lane));
}
__device__ __forceinline__ void ld_row3_h(h4* dst, const uint16_t* row) {
  const int lane = lane_id_fresh();
#pragma unroll
  for (int i = 0; i < 3; ++i) dst[i] = __builtin_nontemporal_load((const h4*)(row + 256 * i + 4 * lane));
}

template <bool Q8, bool H16>
__device__ __forceinline__ void load_row768(WRegs<Q8, H16>& R, int slot, const Weights& w, int l, int m, int r) {
  r = __builtin_amdgcn_readfirstlane(r);  // one row per wave: its offset in scalar registers
  if constexpr (H16) {
    ld_row3_h(&R.r[3 * slot], f16_mat(w, l, m) + (size_t)r * D);
  } else if constexpr (!Q8) {
    ld_row3(&R.r[3 * slot], f32_mat(w, l, m) + (size_t)r * D);
  } else {
    q8_load_row768q(R.c[slot], R.sc[slot], q8_codes(w, l, m), q8_scales(w, l, m), r);
  }
}

// fp32 MLP-projection weights of a regular unit in LDS: [wave 1..7][unit k < 4]
// [pass p < 3] one float4 per lane, written by direct global-to-LDS loads.
struct PrLds {
  f4 w[NCW][UPW][3][64];
};
static_assert(sizeof(PrLds) >= (size_t)FT * 128, "head units stage their output-projection rows in this space");
__device__ __forceinline__ const f4& pr_w(const PrLds& P, int wave, int k, int p) {
  return P.w[wave - 1][k][p][lane_id()];
}
// binary16: a unit's 12 group dots of 64 halves sit contiguously at the start of its
// fp32 space (group dot kk at byte 128 kk), so pass p of lane (qq, j) reads the 8
// bytes at 512 p + 8 lane.
__device__ __forceinline__ char* pr_unit(PrLds& P, int wave, int k) { return (char*)&P.w[wave - 1][k][0][0]; }
__device__ __forceinline__ f4 pr_w16(PrLds& P, int wave, int k, int p) {
  return widen(*(const h4*)(pr_unit(P, wave, k) + 512 * p + 8 * lane_id()));
}

// All units of a regular compute wave for block l.
template <bool Q8, bool H16>
__device__ __forceinline__ void load_block(WRegs<Q8, H16>& R, PrLds& P, const Weights& w, int l, const Units& U,
                                           int wave) {
  const int lane = lane_id_fresh();
#pragma unroll
  for (int k = 0; k < UPW; ++k) {
    const int r = qkv_row(U.X, min(U.qkv(k), 192 * U.nh - 1));
    load_row768<Q8, H16>(R, k, w, l, M_QKV, r);
    R.b[k] = small_p(w, l, sp::B_QKV)[r];
  }
#pragma unroll
  for (int k = 0; k < UPW; ++k) {
    const int r = GS * U.X + min(U.cw + U.cwn * k, GS - 1);
    load_row768<Q8, H16>(R, UPW + k, w, l, M_FC, r);
    R.b[UPW + k] = small_p(w, l, sp::B_FC)[r];
  }
  // MLP projection.  fp32: row pair u (< 384) = rows 2u, 2u+1 over the XCD's slice;
  // pass p, quarter qq takes group dot kk = 4p+qq: row 2u + kk/6, slice group kk%6.
  // binary16: the same group dots, 1536 bytes per unit: one 16-byte copy per lane for
  // kk < 8 (8 lanes a group dot), then two 4-byte copies for kk = 8, 9 and 10, 11
  // (32 lanes a group dot).
  // int8: unit n = 16u + lane/4 (< 6*768): output n/6, group 6X + n%6.
#pragma unroll
  for (int k = 0; k < UPW; ++k) {
    if constexpr (H16) {
      const int u = min(U.cw + U.cwn * k, D / 2 - 1);
      const uint16_t* W = f16_mat(w, l, M_PR);
      auto gd = [&](int kk) { return W + (size_t)(2 * u + kk / GPS) * F + 64 * (GPS * U.X + kk % GPS); };
      char* dst = pr_unit(P, wave, k);
      __builtin_amdgcn_global_load_lds((const void*)(gd(lane / 8) + 8 * (lane % 8)),
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        __builtin_amdgcn_global_load_lds((const void*)(gd(8 + 2 * b + lane / 32) + 2 * (lane % 32)),
                                         (__attribute__((address_space(3))) void*)(dst + 1024 + 256 * b), 4, 0, 0);
    } else if constexpr (!Q8) {
      const int u = min(U.cw + U.cwn * k, D / 2 - 1);
      const float* W = f32_mat(w, l, M_PR);
      const int qq = lane / 16, j = lane % 16;
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        const int kk = 4 * p + qq, row = 2 * u + kk / GPS, g = GPS * U.X + kk % GPS;
        __builtin_amdgcn_global_load_lds((const void*)(W + (size_t)row * F + 64 * g + 4 * j),
                                         (__attribute__((address_space(3))) void*)&P.w[wave - 1][k][p][0], 16, 0, 0);
      }
    } else {
      const int u = min(U.cw + U.cwn * k, GPS * D / 16 - 1);
      const int n = 16 * u + lane / 4, i = n / GPS, g = GPS * U.X + n % GPS;
      R.c[2 * UPW + k] = __builtin_nontemporal_load((const i4*)(q8_codes(w, l, M_PR) + (size_t)i * F + 64 * g + 16 * (lane % 4)));
      R.sc[2 * UPW + k] = q8_scales(w, l, M_PR)[(size_t)i * NG_PR + g];
    }
  }
}

// Output projection of head h on a head unit.  Thread t holds half dots
// hd = t + 512k (k < 3): output i = hd/2, inputs 64h + 32(hd%2) + 0..31 of the
// head, i.e. the two halves of an output sit in adjacent lanes.  fp32: f4 slots
// 8k..8k+7; int8: i4 slots 2k, 2k+1 and the output's group scale sc[k].
// Loading: for each k the 256 rows' 64 head columns are copied into LDS with
// coalesced direct loads (rows are contiguous 256 / 64-byte segments), then each
// thread reads its 128 / 32 contiguous bytes (binary16: 64) from there (a thread's half dot is
// one row segment, which a per-lane global load would fetch as scattered 16-byte
// pieces).  Uses `stage` (>= 64 KB of LDS) as scratch; every thread must call it.
__device__ __forceinline__ int o_half(int k) { return (int)threadIdx.x + FT * k; }
template <bool Q8, bool H16>
__device__ __forceinline__ void load_o_head(WRegs<Q8, H16>& R, char* stage, const Weights& w, int l, int h) {
  constexpr int ELEM = Q8 ? 1 : H16 ? 2 : 4;      // bytes of one weight
  constexpr int SEG = 32 * ELEM;                  // bytes of one half dot
  constexpr int CHUNK = (FT / 2) * 2 * SEG;       // 256 rows x 64 columns
  constexpr int ITERS = CHUNK / (FT * 16);
  static_assert(ITERS * FT * 16 == CHUNK, "chunk");
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = lane_id_fresh();
  const char* base = Q8 ? (const char*)q8_codes(w, l, M_O)
                    : H16 ? (const char*)f16_mat(w, l, M_O) : (const char*)f32_mat(w, l, M_O);
#pragma unroll
  for (int k = 0; k < O_HALF_PER_THREAD; ++k) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int off0 = (it * FT + wave * 64) * 16;  // wave-uniform LDS byte offset
      const int off = off0 + lane * 16;
      const int row = (FT / 2) * k + off / (2 * SEG), colb = off % (2 * SEG);
      __builtin_amdgcn_global_load_lds((const void*)(base + ((size_t)row * D + DH * h) * ELEM + colb),
                                       (__attribute__((address_space(3))) void*)(stage + off0), 16, 0, 0);
    }
    __syncthreads();  // every wave's copies have landed
    const char* mine = stage + (size_t)threadIdx.x * SEG;
    if constexpr (H16) {
#pragma unroll
      for (int j = 0; j < 8; ++j) R.r[8 * k + j] = *(const h4*)(mine + 8 * j);
    } else if constexpr (!Q8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) R.r[8 * k + j] = *(const f4*)(mine + 16 * j);
    } else {
      R.c[2 * k] = *(const i4*)mine;
      R.c[2 * k + 1] = *(const i4*)(mine + 16);
      const int i = o_half(k) >> 1;
      R.sc[k] = q8_scales(w, l, M_O)[(size_t)i * H + h];
    }
    __syncthreads();  // the stage is free again
  }
}

// Head row r (clamped to the last row) into head slot s.
template <bool Q8, bool H16>
__device__ __forceinline__ void load_head(WRegs<Q8, H16>& R, const Weights& w, int s, int r) {
  r = __builtin_amdgcn_readfirstlane(min(r, V - 1));
  if constexpr (H16) {
    ld_row3_h(&R.r[3 * s], f16_mat(w, 0, M_HEAD) + (size_t)r * D);
  } else if constexpr (!Q8) {
    ld_row3(&R.r[3 * s], w.wte + (size_t)r * D);
  } else {
    q8_load_row768q(R.c[s], R.sc[s], q8_codes(w, 0, M_HEAD), q8_scales(w, 0, M_HEAD), r);
  }
}
// Set 0 fills its head slots while set 1 computes the last block.  It waits ~1.8 µs
// first (s_sleep: 64 clocks a unit), so that the 50 MB burst does not meet set 1's
// reduce-scatter of block 10's MLP terms and the start of block 11: fp32 125.5 -> 125.05
// µs (binary32 and binary16; int8 0.25 µs slower with it, so it does not wait).
__device__ __forceinline__ void head_fill_wait() { __builtin_amdgcn_s_sleep(64); }
template <bool Q8, bool H16>
__device__ __forceinline__ void load_head_slots(WRegs<Q8, H16>& R, const Weights& w, HeadRows hr) {
#pragma unroll
  for (int s = 0; s < nhs<Q8>(); ++s) load_head<Q8, H16>(R, w, s, hr.first + s * HEAD_SET_WAVES);
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
  float xs[D];          // block input x (all-gather), x12 for the head
  float x1s[D];         // x1 (all-gather; a buffer of its own: waves 1..7 may still read xs)
  float xn[D];          // LayerNorm output (fp32: of x; int8: of x or x1)
  float lntmp[D];       // fp32: LayerNorm output of x1; int8: LayerNorm scratch
  float att[DH];        // attention output of a head unit
  float xg[GS];         // the XCD's GELU slice
  float rs[NG_PR * RSN];  // reduce-scatter terms
  float lnp[4][D];      // LayerNorm parameters of the unit's next block: ln1 gamma, beta, ln2 gamma, beta
  float lnf[2][D];      // final LayerNorm gamma, beta
  int8_t xc[F];         // int8 path: input codes (by input index)
  float xsc[64];        // int8 path: input scales (by group)
  union {
    AttnSmem at;        // head units
    PrLds pr;           // regular units, fp32
  };
};
// int8 path: the candidate table of the workgroup LayerNorm sums.  It shares the
// union: int8 regular units keep no weights in LDS, and head units take a
// LayerNorm only after their last attention.
__device__ __forceinline__ float* seq_tab(FusedSmem& S) { return reinterpret_cast<float*>(&S.pr); }
static_assert(sizeof(PrLds) >= SEQ_TAB_FLOATS * sizeof(float), "LayerNorm candidate table");

// Per-workgroup constants.
struct Ctx {
  uint32_t E;  // this launch's epoch
  int X;       // XCD
  int set;     // 0: blocks 0, 2, ...; 1: blocks 1, 3, ...
  int q;       // rank inside the XCD's set
  int nh;      // heads of the XCD
  bool head;   // head unit (q < nh): head X + 8q
  u64* loc;    // this XCD's local words, block 0
  u64* glb;    // global words, block 0
};
// The head rows of wave `wave` of this workgroup: index i < 1,024 within its set.
template <bool Q8>
__device__ __forceinline__ HeadRows head_rows_of(const Ctx& c, int wave) {
  const int i = wave * (GRID / 2) + ((int)blockIdx.x % NX) + NX * c.q;
  constexpr int n0 = head_n0<Q8>();
  return c.set == 0 ? HeadRows{i, n0} : HeadRows{n0 * HEAD_SET_WAVES + i, HEAD_TOTAL - n0};
}
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
  stage_vec(S.lnp[0], small_p(w, l, sp::LN1_G));
  stage_vec(S.lnp[1], small_p(w, l, sp::LN1_B));
  stage_vec(S.lnp[2], small_p(w, l, sp::LN2_G));
  stage_vec(S.lnp[3], small_p(w, l, sp::LN2_B));
}

// x = wte[token] + wpe[pos] into LDS (if xs) ; lanes < RSN return element RSN*q + lane.
// TOKP (a generation step): the token is the one the previous step's greedy choice
// left in the workspace header, not the launch argument.
template <bool TOKP>
__device__ __forceinline__ float embed(const FusedArgs& a, float* xs, int q) {
  const int lane = lane_id();
  const uint32_t tok = TOKP ? min(ld32(&a.header[HDR_WORD_NEXT_TOKEN]), (uint32_t)V - 1) : a.token;
  if (xs) {
#pragma unroll
    for (int j = 0; j < 12; ++j) {
      const int i = lane + 64 * j;
      xs[i] = a.w.wte[(size_t)tok * D + i] + a.w.wpe[(size_t)a.pos * D + i];
    }
  }
  const int o = RSN * q + min(lane, RSN - 1);
  return a.w.wte[(size_t)tok * D + o] + a.w.wpe[(size_t)a.pos * D + o];
}

// Set 1 defers its first weight loads until set 0 has published its first QKV
// rows: at launch both sets would otherwise share the HBM bandwidth and delay block
// 0, while set 1's weights are only needed a block later.
__device__ __forceinline__ void defer_set1(const Ctx& c, uint32_t* hdr) {
  if (c.set == 0) return;
  float v[1];
  poll<1, true>(loc_of(c, 0) + LO_QKV, 1, [](int k) { return k; }, c.E, v, hdr);
}

// Reduce-scatter of block l's MLP projection by a unit of the set that computes
// block l+1: wave 0 forms x_{l+1}[o] = x1_l[o] + (sum + bias) and publishes it into
// the XCD's copy (rs_pr); lanes < RSN return it.  int8 (48 group terms per output):
// every wave first polls its share of the terms into LDS (rs_pr_poll), and rs_pr
// adds them after a workgroup barrier.  fp32 (8 slice terms): rs_pr reads them
// itself (rs_lanes), so the other waves take no part.
template <bool Q8>
__device__ __forceinline__ void rs_pr_poll(const FusedArgs& a, FusedSmem& S, const Ctx& c, int l, int wave) {
  if constexpr (Q8) rs_poll_part<NG_PR>(glb_of(c, l) + GL_P, c.q, c.E, S.rs, a.header, wave);
}
// The unit's share of x1 of block l (lanes < RSN), published inside the XCD in the
// middle of block l: the wave that takes the reduce-scatter reads it before it polls
// the MLP terms, so this read is off the path that waits for them.
__device__ __forceinline__ float x1_share(const FusedArgs& a, const Ctx& c, int l) {
  float x1[1];
  poll<1, true>(loc_of(c, l) + LO_X1 + RSN * c.q, RSN, [](int k) { return k; }, c.E, x1, a.header);
  return x1[0];
}
template <bool Q8, bool CAP>
__device__ __forceinline__ float rs_pr(const FusedArgs& a, FusedSmem& S, const Ctx& c, int l, float bpr, float x1) {
  const int lane = lane_id();
  float y;
  if constexpr (Q8) y = rs_sum<NG_PR>(S.rs);
  else y = rs_lanes<NX>(glb_of(c, l) + GL_P, c.q, c.E, a.header);
  float xr = 0.0f;
  if (lane < RSN) {
    const int o = RSN * c.q + lane;
    y = y + bpr;
    if (CAP && c.X == 0) ((float*)(a.capture + cap_offset(l, M_PR) + cap_item(M_PR).y))[o] = y;
    xr = x1 + y;
    st_loc(loc_of(c, l) + LO_X2 + o, pack(xr, c.E));
  }
  return xr;
}
// Reduce-scatter of block l's output projection: x1[o] = x[o] + (sum + bias).
template <bool Q8, bool CAP>
__device__ __forceinline__ float rs_o(const FusedArgs& a, FusedSmem& S, const Ctx& c, int l, float xr, float bo) {
  const int lane = lane_id();
  float y = rs_lanes<H>(glb_of(c, l) + GL_O, c.q, c.E, a.header);
  float x1 = 0.0f;
  if (lane < RSN) {
    const int o = RSN * c.q + lane;
    y = y + bo;
    if (CAP && c.X == 0) ((float*)(a.capture + cap_offset(l, M_O) + cap_item(M_O).y))[o] = y;
    x1 = xr + y;
    st_loc(loc_of(c, l) + LO_X1 + o, pack(x1, c.E));
  }
  return x1;
}

// int8: quantize groups g0, g0+gstep, ... (< g1) of src (LDS, indexed from group
// gsrc0) into xc/xsc by input index, one group per compute wave (waves 1..7).
__device__ __forceinline__ void quantize_groups(FusedSmem& S, const float* src, int gsrc0, int g0, int g1, int wave) {
  const int lane = lane_id();
  for (int g = g0 + (wave - 1); g < g1; g += NCW) {
    float s;
    const int qv = quant_lane(src[(g - gsrc0) * 64 + lane], s);
    S.xc[g * 64 + lane] = (int8_t)qv;
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

// ---- the tied head -------------------------------------------------------------
// Head rows of a wave (hr): the first NS slots were loaded ahead; each slot is
// refilled with the row NS further on as soon as it has been used.  Rows past the
// vocabulary compute on the last row and store to the sink.
template <bool Q8, bool CAP, bool H16>
__device__ __forceinline__ void head_rows(const FusedArgs a, FusedSmem& S, WRegs<Q8, H16>& R, HeadRows hr,
                                          float* sinkf) {
  constexpr int NMAX = head_nmax<Q8>();
  const int lane = lane_id();
  constexpr int NS = nhs<Q8>();
  f4 x[3];
  if constexpr (!Q8) {
    load_frag<3>(x, S.xs);
    layernorm_frag(x, S.lnf[0], S.lnf[1]);
  }
  if constexpr (!Q8) {
    // four rows at a time: their lane partials reduced together (wave_treduce, the
    // adds of dot_slots' wave_sum); lane t stores row k0 + treduce_out<4>(t)
    constexpr int HR = 4;
    static_assert(NS % HR == 0, "head row groups");
#pragma unroll
    for (int k0 = 0; k0 < NMAX; k0 += HR) {
      // keep the loads in slot order: at most NHS rows in flight per wave
      __builtin_amdgcn_sched_barrier(0);
      if (k0 < hr.n) {  // a uniform guard, not a break: the loop stays fully unrolled
        float lp[HR];
#pragma unroll
        for (int u = 0; u < HR; ++u) lp[u] = dot_slots_lane<H16>(R, 3 * ((k0 + u) % NS), x);
        const float y = wave_treduce<HR>(lp);
        const int k = k0 + treduce_out<HR>(lane & 15), r = hr.first + k * HEAD_SET_WAVES;
        *(k < hr.n && r < V ? a.logits + r : sinkf) = y;  // a row past hr.n used a stale slot
#pragma unroll
        for (int u = 0; u < HR; ++u) {
          const int ku = k0 + u;
          if (ku + NS < hr.n) load_head<Q8, H16>(R, a.w, ku % NS, hr.first + (ku + NS) * HEAD_SET_WAVES);
        }
        if (k0 + HR == NS && lane == 0 && (threadIdx.x >> 6) == 1) stamp(a.trace, 57);
      }
    }
  } else {
    // int8: an int8 row is a long dependent chain for few bytes, so HG rows are
    // evaluated together (their chains overlap), then stored and their slots refilled
    constexpr int HG = 4;
    static_assert(NS % HG == 0, "head groups");
#pragma unroll
    for (int k0 = 0; k0 < NMAX; k0 += HG) {
      __builtin_amdgcn_sched_barrier(0);
      if (k0 < hr.n) {
        // the group's rows together (q8_dot768q_x4): lane u < 4 returns row k0 + u; a
        // row past hr.n computes on a stale slot and is not stored
        i4 wc[HG];
        float sw[HG];
        int32_t* ca[HG];
#pragma unroll
        for (int u = 0; u < HG; ++u) {
          const int k = k0 + u, r = hr.first + k * HEAD_SET_WAVES, s = k % NS;
          wc[u] = R.c[s];
          sw[u] = R.sc[s];
          ca[u] = CAP && k < hr.n && r < V
                      ? (int32_t*)(a.capture + cap_offset(0, M_HEAD) + cap_item(M_HEAD).acc) + (size_t)r * 12
                      : nullptr;
        }
        const float y = q8_dot768q_x4(wc, sw, S.xc, S.xsc, ca);
        if (lane < HG && k0 + lane < hr.n) {
          const int r = hr.first + (k0 + lane) * HEAD_SET_WAVES;
          if (CAP && r < V) ((float*)(a.capture + cap_offset(0, M_HEAD) + cap_item(M_HEAD).y))[r] = y;
          *(r < V ? a.logits + r : sinkf) = y;
        }
#pragma unroll
        for (int u = 0; u < HG; ++u) {
          const int k = k0 + u, r = hr.first + k * HEAD_SET_WAVES, s = k % NS;
          if (k + NS < hr.n) load_head<Q8, H16>(R, a.w, s, r + NS * HEAD_SET_WAVES);
        }
      }
      if (k0 + HG == NS && lane == 0 && (threadIdx.x >> 6) == 1) stamp(a.trace, 57);
    }
  }
}

// ---- regular units -------------------------------------------------------------
// Wave 0 receives (reduce-scatters, all-gathers) and holds no weights; it also
// takes the block's two LayerNorms once for the workgroup (fp32: layernorm_frag on x
// and x1 gathered straight into registers, written to xn and lntmp; int8: with the
// whole workgroup, layernorm_seq_wg).  Waves 1..7
// compute from registers (and the fp32 MLP weights from LDS).  The two roles meet
// at the same sequence of workgroup barriers.
template <bool Q8, bool CAP, bool TOKP, bool H16>
__device__ __forceinline__ void regular_io(const FusedArgs& a, FusedSmem& S, const Ctx& c, WRegs<Q8, H16>& R) {
  const int lane = lane_id();
  uint32_t* hdr = a.header;
  const uint32_t E = c.E;
  const bool cap0 = CAP && c.X == 0 && c.q == c.nh;  // one regular unit captures LayerNorm-output inputs
  const bool capx = CAP && c.q == c.nh;              // one per XCD captures its GELU slice
  const int o = RSN * c.q + min(lane, RSN - 1);
  const int l0 = c.set;
  stage_ln(S, a.w, l0);
  stage_vec(S.lnf[0], a.w.small + sp::LNF_G);
  stage_vec(S.lnf[1], a.w.small + sp::LNF_B);
  float bo = small_p(a.w, l0, sp::B_O)[o];
  float bpr = l0 > 0 ? small_p(a.w, l0 - 1, sp::B_PR)[o] : 0.0f;
  float xr;
  wg_barrier();  // B0
  for (int l = l0; l < L; l += 2) {
    u64* loc = loc_of(c, l);
    float x1p = 0.0f;
    if (l > 0) {
      x1p = x1_share(a, c, l - 1);
      rs_pr_poll<Q8>(a, S, c, l - 1, 0);
    }
    dstamp(a.trace, l, 52);
    wg_barrier();  // BA: the reduce-scatter terms are in LDS
    dstamp(a.trace, l, 53);
    f4 xf[3];  // fp32: the block input in the lane-fragment layout
    if (l == 0) {
      xr = embed<TOKP>(a, S.xs, c.q);
      if constexpr (!Q8) load_frag<3>(xf, S.xs);
    } else {
      xr = rs_pr<Q8, CAP>(a, S, c, l - 1, bpr, x1p);
      dstamp(a.trace, l, 54);
      if constexpr (Q8) gather<12>(loc_of(c, l - 1) + LO_X2, E, S.xs, hdr);
      else gather_frag(loc_of(c, l - 1) + LO_X2, E, xf, hdr);
    }
    if (lane == 0) stamp(a.trace, 1 + 4 * l);
    if constexpr (Q8) {
      wg_barrier();  // the block input is in LDS
      layernorm_seq_wg<1>(S.xs, S.lnp[0], S.lnp[1], S.xn, S.lntmp, seq_tab(S), S.xc, S.xsc);
    } else {
      layernorm_frag(xf, S.lnp[0], S.lnp[1]);  // once for the workgroup
      store_frag<3>(S.xn, xf);
    }
    wg_barrier();  // B1: QKV (int8: its input codes are in LDS)
    if constexpr (Q8) {
      if (cap0) capture_input(a, S, l, M_QKV, S.xn, 0, D, lane, 64);
    }
    xr = rs_o<Q8, CAP>(a, S, c, l, xr, bo);
    dstamp(a.trace, l, 56);
    if constexpr (Q8) {
      gather<12>(loc + LO_X1, E, S.x1s, hdr);
      if (lane == 0) stamp(a.trace, 3 + 4 * l);
      wg_barrier();  // x1 is in LDS
      layernorm_seq_wg<1>(S.x1s, S.lnp[2], S.lnp[3], S.xn, S.lntmp, seq_tab(S), S.xc, S.xsc);
    } else {
      gather_frag(loc + LO_X1, E, xf, hdr);
      if (lane == 0) stamp(a.trace, 3 + 4 * l);
      layernorm_frag(xf, S.lnp[2], S.lnp[3]);
      store_frag<3>(S.lntmp, xf);
    }
    wg_barrier();  // B3: FC (int8: its input codes are in LDS)
    if constexpr (Q8) {
      if (cap0) capture_input(a, S, l, M_FC, S.xn, 0, D, lane, 64);
    }
    gather<GS / 64>(loc + LO_G, E, S.xg, hdr);
    if (lane == 0) stamp(a.trace, 4 + 4 * l);
    wg_barrier();  // B4: MLP projection
    if constexpr (Q8) {
      wg_barrier();
      if (capx) capture_input(a, S, l, M_PR, S.xg, GS * c.X, GS * (c.X + 1), lane, 64);
    }
    // the next block of this set: its LayerNorm parameters and reduce-scatter biases
    const int ln = l + 2;
    if (ln < L) {
      stage_ln(S, a.w, ln);
      bo = small_p(a.w, ln, sp::B_O)[o];
    }
    if (ln - 1 < L) bpr = small_p(a.w, ln - 1, sp::B_PR)[o];
  }
  // the tied head: set 0 reduces block 11's MLP projection, both gather x12.  Binary32
  // and binary16: set 0's input wave fills its head slots now, while set 1 computes
  // block 11 (they land long before its block-11 polls, which would otherwise return
  // behind them); otherwise the input wave fills them when the head starts (int8:
  // filling them here measured 4.7 µs slower).
  if (!Q8 && c.set == 0) {
    head_fill_wait();
    load_head_slots<Q8, H16>(R, a.w, head_rows_of<Q8>(c, 0));
  }
  float x1p = 0.0f;
  if (c.set == 0) {
    x1p = x1_share(a, c, L - 1);
    rs_pr_poll<Q8>(a, S, c, L - 1, 0);
  }
  wg_barrier();  // BT
  if (c.set == 0) rs_pr<Q8, CAP>(a, S, c, L - 1, bpr, x1p);
  gather<12>(loc_of(c, L - 1) + LO_X2, E, S.xs, hdr);
  if (lane == 0) stamp(a.trace, 49);
}

template <bool Q8, bool CAP, bool H16>
__device__ __forceinline__ void regular_compute(const FusedArgs& a, FusedSmem& S, const Ctx& c, WRegs<Q8, H16>& R,
                                                int wave) {
  const int lane = lane_id();
  const uint32_t E = c.E;
  u64* sinkw = a.sinkw + ((size_t)blockIdx.x * 8 + wave) * 16;
  float* sinkf = (float*)(sinkw + 8);
  Units U;
  U.X = c.X;
  U.nh = c.nh;
  U.cwn = NCW * (NQ - c.nh);
  U.cw = (wave - 1) * (NQ - c.nh) + (c.q - c.nh);
  const int l0 = c.set;
  defer_set1(c, a.header);
  // Binary32: set 0's block-0 stream starts ~0.2 µs after the head units' output-projection
  // staging, which the block-0 attention waits for (124.8 -> 124.5 µs; the int8 and
  // binary16 steps are 0.5 µs slower with it, so they do not wait).
  if (!Q8 && !H16 && c.set == 0) __builtin_amdgcn_s_sleep(8);
  load_block<Q8, H16>(R, S.pr, a.w, l0, U, wave);
  wg_barrier();  // B0
  for (int l = l0; l < L; l += 2) {
    u64* loc = loc_of(c, l);
    u64* glb = glb_of(c, l);
    if (l > 0) rs_pr_poll<Q8>(a, S, c, l - 1, wave);
    // The block's weights (registers and direct-to-LDS copies) landed during the
    // wait: retire them here, so later reads of them wait on no store of this block.
    wave_vmem_sync();
    wg_barrier();  // BA
    if constexpr (Q8) {
      wg_barrier();
      layernorm_seq_wg<0>(S.xs, S.lnp[0], S.lnp[1], S.xn, S.lntmp, seq_tab(S), S.xc, S.xsc);
    }
    wg_barrier();  // B1: QKV
    if (wave == 1) dstamp(a.trace, l, 59);
    {
      f4 x[3];
      if constexpr (!Q8) load_frag<3>(x, S.xn);
      if (wave == 1) dstamp(a.trace, l, 60);
      if constexpr (!Q8 && FUSED_TRED) {
        // the four rows reduced together; lanes 0..3 hold rows 0, 1, 3, 2 and store them
        int k;
        const float y = rows_treduce<0>(R, x, k);
        if (lane < UPW) {
          const int n = U.qkv(k);
          const bool own = n < 192 * U.nh;
          const int r = qkv_row(U.X, own ? n : 0);
          st_loc(own ? loc + LO_QKV + n : sinkw, pack(y, E));
          *(own && r >= D ? a.cache + ((size_t)a.pos * L + l) * KV_ROW + (r - D) : sinkf) = y;
        }
      } else if constexpr (Q8 && FUSED_TRED) {
        // the four rows together (q8_dot768q_x4): lanes 0..3 hold rows 0..3
        i4 wc[UPW];
        float sw[UPW], bb[UPW];
        int32_t* ca[UPW];
#pragma unroll
        for (int k = 0; k < UPW; ++k) {
          const int n = U.qkv(k);
          const bool own = n < 192 * U.nh;
          wc[k] = R.c[k];
          sw[k] = R.sc[k];
          bb[k] = R.b[k];
          asm volatile("" : "+v"(bb[k]));
          ca[k] = CAP && own ? (int32_t*)(a.capture + cap_offset(l, M_QKV) + cap_item(M_QKV).acc) +
                                   (size_t)qkv_row(U.X, n) * 12
                             : nullptr;
        }
        const int k = lane & 3;
        const float y = q8_dot768q_x4(wc, sw, S.xc, S.xsc, ca) + (k == 0 ? bb[0] : k == 1 ? bb[1] : k == 2 ? bb[2] : bb[3]);
        if (lane < UPW) {
          const int n = U.qkv(k);
          const bool own = n < 192 * U.nh;
          const int r = qkv_row(U.X, own ? n : 0);
          st_loc(own ? loc + LO_QKV + n : sinkw, pack(y, E));
          *(own && r >= D ? a.cache + ((size_t)a.pos * L + l) * KV_ROW + (r - D) : sinkf) = y;
          if (CAP && own) ((float*)(a.capture + cap_offset(l, M_QKV) + cap_item(M_QKV).y))[r] = y;
        }
      } else
#pragma unroll
      for (int k = 0; k < UPW; ++k) {
        const int n = U.qkv(k);
        const bool own = n < 192 * U.nh;
        const int r = qkv_row(U.X, own ? n : 0);
        float y;
        if constexpr (!Q8) {
          y = dot_slots(R, 3 * k, x);
        } else {
          int32_t* ca = CAP && own ? (int32_t*)(a.capture + cap_offset(l, M_QKV) + cap_item(M_QKV).acc) + (size_t)r * 12
                                   : nullptr;
          y = q8_dot768q(R.c[k], R.sc[k], S.xc, S.xsc, ca);
        }
        y = y + R.b[k];
        st_loc(own ? loc + LO_QKV + n : sinkw, pack(y, E));
        *(own && r >= D ? a.cache + ((size_t)a.pos * L + l) * KV_ROW + (r - D) : sinkf) = y;
        if (CAP && own && lane == 0) ((float*)(a.capture + cap_offset(l, M_QKV) + cap_item(M_QKV).y))[r] = y;
      }
    }
    if (wave == 1 && lane == 0) stamp(a.trace, 2 + 4 * l);
    if constexpr (Q8) {
      wg_barrier();
      layernorm_seq_wg<0>(S.x1s, S.lnp[2], S.lnp[3], S.xn, S.lntmp, seq_tab(S), S.xc, S.xsc);
    }
    wg_barrier();  // B3: FC
    {
      f4 x[3];
      if constexpr (!Q8) load_frag<3>(x, S.lntmp);
      if constexpr (!Q8 && FUSED_TRED) {
        int k;
        const float y = rows_treduce<UPW>(R, x, k);
        const float gy = gelu_f32(y);
        if (lane < UPW) {
          const int n = U.cw + U.cwn * k;
          st_loc(n < GS ? loc + LO_G + n : sinkw, pack(gy, E));
        }
      } else if constexpr (Q8 && FUSED_TRED) {
        i4 wc[UPW];
        float sw[UPW], bb[UPW];
        int32_t* ca[UPW];
#pragma unroll
        for (int k = 0; k < UPW; ++k) {
          const int n = U.cw + U.cwn * k;
          wc[k] = R.c[UPW + k];
          sw[k] = R.sc[UPW + k];
          bb[k] = R.b[UPW + k];
          asm volatile("" : "+v"(bb[k]));
          ca[k] = CAP && n < GS ? (int32_t*)(a.capture + cap_offset(l, M_FC) + cap_item(M_FC).acc) +
                                      (size_t)(GS * U.X + n) * 12
                                : nullptr;
        }
        const int k = lane & 3;
        const float y = q8_dot768q_x4(wc, sw, S.xc, S.xsc, ca) + (k == 0 ? bb[0] : k == 1 ? bb[1] : k == 2 ? bb[2] : bb[3]);
        const float gy = gelu_tanh(y);
        if (lane < UPW) {
          const int n = U.cw + U.cwn * k;
          const bool own = n < GS;
          st_loc(own ? loc + LO_G + n : sinkw, pack(gy, E));
          if (CAP && own) ((float*)(a.capture + cap_offset(l, M_FC) + cap_item(M_FC).y))[GS * U.X + n] = y;
        }
      } else
#pragma unroll
      for (int k = 0; k < UPW; ++k) {
        const int n = U.cw + U.cwn * k;
        const bool own = n < GS;
        const int r = GS * U.X + (own ? n : 0);
        float y;
        if constexpr (!Q8) {
          y = dot_slots(R, 3 * (UPW + k), x);
        } else {
          int32_t* ca = CAP && own ? (int32_t*)(a.capture + cap_offset(l, M_FC) + cap_item(M_FC).acc) + (size_t)r * 12
                                   : nullptr;
          y = q8_dot768q(R.c[UPW + k], R.sc[UPW + k], S.xc, S.xsc, ca);
        }
        y = y + R.b[UPW + k];
        const float gy = Q8 ? gelu_tanh(y) : gelu_f32(y);
        st_loc(own ? loc + LO_G + n : sinkw, pack(gy, E));
        if (CAP && own && lane == 0) ((float*)(a.capture + cap_offset(l, M_FC) + cap_item(M_FC).y))[r] = y;
      }
    }
    wg_barrier();  // B4: MLP projection
    if (wave == 1) dstamp(a.trace, l, 62);
    if constexpr (Q8) {
      quantize_groups(S, S.xg, GPS * c.X, GPS * c.X, GPS * (c.X + 1), wave);
      wg_barrier();
    }
    if constexpr (!Q8) {
      // every LDS read of the phase first (the slice's inputs of the three passes and
      // the four units' weights), so the dots wait for LDS once
      const int qq = lane / 16, j = lane % 16;
      f4 xv[3], wv[UPW][3];
#pragma unroll
      for (int p = 0; p < 3; ++p) xv[p] = *(const f4*)(S.xg + 64 * ((4 * p + qq) % GPS) + 4 * j);
#pragma unroll
      for (int k = 0; k < UPW; ++k)
#pragma unroll
        for (int p = 0; p < 3; ++p) wv[k][p] = H16 ? pr_w16(S.pr, wave, k, p) : pr_w(S.pr, wave, k, p);
#if FUSED_MLP_TRED
      // The four units' group dots of a pass reduced together (row_treduce: the adds of
      // dot_q16's row16_sum): g[p] in lane t of row qq holds group kk = 4p + qq of unit
      // treduce_out<4>(t).  The slice sums then run in group order in the lanes of row
      // 0 for all four units at once, each group moved there from its row: row 2u adds
      // groups 0..5, row 2u+1 groups 6..11 (pr_row's order).
      static_assert(UPW == 4 && GPS == 6, "MLP phase layout");
      float g[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) {
        float lp[UPW];
#pragma unroll
        for (int k = 0; k < UPW; ++k) {
          float acc = 0.0f;
          acc = fmaf(wv[k][p].x, xv[p].x, acc);
          acc = fmaf(wv[k][p].y, xv[p].y, acc);
          acc = fmaf(wv[k][p].z, xv[p].z, acc);
          acc = fmaf(wv[k][p].w, xv[p].w, acc);
          lp[k] = acc;
        }
        g[p] = row_treduce<UPW>(lp);
      }
      float p0 = g[0];
      p0 = p0 + row1_to_row0(g[0]);
      p0 = p0 + row2_to_row0(g[0]);
      p0 = p0 + row3_to_row0(g[0]);
      p0 = p0 + g[1];
      p0 = p0 + row1_to_row0(g[1]);
      float p1 = row2_to_row0(g[1]);
      p1 = p1 + row3_to_row0(g[1]);
      p1 = p1 + g[2];
      p1 = p1 + row1_to_row0(g[2]);
      p1 = p1 + row2_to_row0(g[2]);
      p1 = p1 + row3_to_row0(g[2]);
#pragma unroll
      for (int k = 0; k < UPW; ++k) {
        const int u0 = U.cw + U.cwn * k;
        const bool own = u0 < D / 2;
        const int u = own ? u0 : 0;
        constexpr int TK[4] = {treduce_lane<4>(0), treduce_lane<4>(1), treduce_lane<4>(2), treduce_lane<4>(3)};
        const float a0 = lane_val(p0, TK[k]), a1 = lane_val(p1, TK[k]);
        // lanes 0..31 store row 2u, lanes 32..63 row 2u+1
        const int half = lane >> 5;
        st_sc1(own ? glb + GL_P + (size_t)U.X * D + 2 * u + half : sinkw, pack(half ? a1 : a0, E));
      }
#else
#pragma unroll
      for (int k = 0; k < UPW; ++k) {
        const int u0 = U.cw + U.cwn * k;
        const bool own = u0 < D / 2;
        const int u = own ? u0 : 0;
        float qv[3];
#pragma unroll
        for (int p = 0; p < 3; ++p) qv[p] = dot_q16(wv[k][p], xv[p]);
        auto val = [&](int kk) { return lane_val(qv[kk / 4], 16 * (kk % 4)); };
        float p0 = val(0), p1 = val(GPS);
#pragma unroll
        for (int kk = 1; kk < GPS; ++kk) {
          p0 = p0 + val(kk);
          p1 = p1 + val(GPS + kk);
        }
        // lanes 0..31 store row 2u, lanes 32..63 row 2u+1
        const int half = lane >> 5;
        st_sc1(own ? glb + GL_P + (size_t)U.X * D + 2 * u + half : sinkw, pack(half ? p1 : p0, E));
      }
#endif
    } else {
#pragma unroll
      for (int k = 0; k < UPW; ++k) {
        const int u0 = U.cw + U.cwn * k;
        const bool own = u0 < GPS * D / 16;
        const int n = 16 * (own ? u0 : 0) + lane / 4, i = n / GPS, g = GPS * U.X + n % GPS;
        const i4 xv = *(const i4*)(S.xc + 64 * g + 16 * (lane % 4));
        const int acc = quad_acc(R.c[2 * UPW + k], xv);
        const float t = ((float)acc * R.sc[2 * UPW + k]) * S.xsc[g];
        st_sc1(own ? glb + GL_P + (size_t)g * D + i : sinkw, pack(t, E));
        if (CAP && own && lane % 4 == 0)
          ((int32_t*)(a.capture + cap_offset(l, M_PR) + cap_item(M_PR).acc))[(size_t)i * NG_PR + g] = acc;
      }
    }
    if (wave == 1) dstamp(a.trace, l, 63);
    // this block is done: the weights of the set's next block (or the first head rows).
    // The MLP terms have reached memory before that stream starts: stores still queued
    // behind a wave's weight loads would hold up the other set's reduce-scatter.  The
    // stream then waits a little longer (s_sleep: 64 clocks a unit, ~2.8 µs binary32, ~1.8
    // µs int8), so that its first burst does not meet the other set's reduce-scatter of
    // these terms and the start of the next block; it still has most of a block to land.
    // Measured: fp32 126.7 -> 125.6 µs, int8 208.3 -> 207.1 µs; at 127 units (3.5 µs) the
    // fp32 step is slower (127.9 µs).
    wave_vmem_sync();
    if (l + 2 < L) {
      __builtin_amdgcn_s_sleep(Q8 ? 64 : 100);
      load_block<Q8, H16>(R, S.pr, a.w, l + 2, U, wave);
    }
  }
  // The first head rows, outside the loop, so the slots past the block weights are not
  // live across it.  (Filling the slots whose block rows are used up during set 1's last
  // block, to start its head stream earlier, delays that block's MLP terms: slower.)
  if (!Q8 && c.set == 0) head_fill_wait();
  load_head_slots<Q8, H16>(R, a.w, head_rows_of<Q8>(c, wave));
  if (c.set == 0) rs_pr_poll<Q8>(a, S, c, L - 1, wave);
  wg_barrier();  // BT
}

// ---- head units (head h = X + 8q) ---------------------------------------------------
// Per block: its keys/values j < pos are in LDS; wave 0 takes the unit's
// reduce-scatter of the previous block and polls the XCD's q/k/v of the head;
// attention; all 8 waves compute the head's output-projection terms for the 768
// outputs and publish them; wave 0 then takes the unit's reduce-scatter of x1.
// Keys/values j < pos of head h at block l into LDS (all threads of a head unit).
__device__ __forceinline__ void stage_kv(const FusedArgs& a, FusedSmem& S, int l, int h) {
  const float* cl = a.cache + (size_t)l * KV_ROW + h * DH;
  attn_stage_rows(S.at, [&](int j) { return cl + (size_t)j * CACHE_POS; }, 0, a.pos, 0, FT);
}

template <bool Q8, bool CAP, bool TOKP, bool H16>
__device__ __forceinline__ void head_unit(const FusedArgs& a, FusedSmem& S, const Ctx& c, WRegs<Q8, H16>& R,
                                          int wave) {
  const int lane = lane_id();
  uint32_t* hdr = a.header;
  const uint32_t E = c.E;
  const int h = c.X + NX * c.q, pos = a.pos;
  AttnSmem& sm = S.at;
  const int o = RSN * c.q + min(lane, RSN - 1);
  const int l0 = c.set;
  u64* sinkw = a.sinkw + ((size_t)blockIdx.x * 8 + wave) * 16;
  float bo = 0.0f, bpr = 0.0f, xr = 0.0f;
  if (wave == 0) defer_set1(c, hdr);
  wg_barrier();
  load_o_head<Q8, H16>(R, (char*)&S.pr, a.w, l0, h);
  stage_kv(a, S, l0, h);
  if (wave == 0) {
    stage_vec(S.lnf[0], a.w.small + sp::LNF_G);
    stage_vec(S.lnf[1], a.w.small + sp::LNF_B);
    bo = small_p(a.w, l0, sp::B_O)[o];
    if (l0 > 0) bpr = small_p(a.w, l0 - 1, sp::B_PR)[o];
  }
  wg_barrier();
  for (int l = l0; l < L; l += 2) {
    u64* glb = glb_of(c, l) + GL_O + (size_t)h * D;
    float x1p = 0.0f;
    if (l > 0) {
      if (wave == 0) x1p = x1_share(a, c, l - 1);
      rs_pr_poll<Q8>(a, S, c, l - 1, wave);
      wg_barrier();
    }
    if (wave == 0) {
      dstamp(a.trace, l, 52);
      xr = l == 0 ? embed<TOKP>(a, nullptr, c.q) : rs_pr<Q8, CAP>(a, S, c, l - 1, bpr, x1p);
      if (lane == 0) stamp(a.trace, 1 + 4 * l);
      float v[3];
      poll<3, true>(loc_of(c, l) + LO_QKV + 192 * c.q, 192, [](int k) { return k; }, E, v, hdr);
      dstamp(a.trace, l, 54);
      sm.q[lane] = v[0];
      sm.k[pos][lane] = v[1];
      sm.v[pos][lane] = v[2];
    }
    wg_barrier();
    const float at = Q8 ? attn_compute_seq(sm, pos + 1) : attn_compute<FT>(sm, pos + 1);
    if (wave == 0) {
      S.att[lane] = at;
      if constexpr (Q8) {
        float sx;
        const int qv = quant_lane(at, sx);
        S.xc[lane] = (int8_t)qv;
        if (lane == 0) S.xsc[0] = sx;
        if (CAP) {
          char* base = a.capture + cap_offset(l, M_O);
          const CapLayout cl2 = cap_item(M_O);
          ((float*)(base + cl2.in))[DH * h + lane] = at;
          ((int8_t*)(base + cl2.codes))[DH * h + lane] = (int8_t)qv;
          if (lane == 0) ((float*)(base + cl2.xs))[h] = sx;
        }
      }
      if (lane == 0) stamp(a.trace, 2 + 4 * l);
    }
    wg_barrier();  // attention output in LDS
    // The output-projection terms.  fp32: a half dot is s_j = the fmaf chain over
    // inputs 4j..4j+3 (j < 8 of its half), then ((s0+s1)+(s2+s3)) + ((s4+s5)+(s6+s7)),
    // and the two halves are added across the lane pair: the same value as
    // dot_q16 over the head's 64 inputs (its 16-lane tree, as o_row uses).  int8:
    // the exact group accumulator, then ((float)acc * sw) * sx.
#pragma unroll
    for (int k = 0; k < O_HALF_PER_THREAD; ++k) {
      const int hd = o_half(k), i = hd >> 1, half = hd & 1;
      float t;
      if constexpr (!Q8) {
        const float* av = S.att + 32 * half;
        float sj[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const f4 x = *(const f4*)(av + 4 * j);
          const f4 wv4 = wslot(R, 8 * k + j);
          float acc = 0.0f;
          acc = fmaf(wv4.x, x.x, acc);
          acc = fmaf(wv4.y, x.y, acc);
          acc = fmaf(wv4.z, x.z, acc);
          acc = fmaf(wv4.w, x.w, acc);
          sj[j] = acc;
        }
        const float hs = ((sj[0] + sj[1]) + (sj[2] + sj[3])) + ((sj[4] + sj[5]) + (sj[6] + sj[7]));
        t = hs + dpp_f<DPP_QUAD_1032>(hs);
      } else {
        const int8_t* xv = S.xc + 32 * half;
        const i4 x0 = *(const i4*)xv, x1 = *(const i4*)(xv + 16);
        int acc = 0;
        acc = __builtin_amdgcn_sdot4(R.c[2 * k].x, x0.x, acc, false);
        acc = __builtin_amdgcn_sdot4(R.c[2 * k].y, x0.y, acc, false);
        acc = __builtin_amdgcn_sdot4(R.c[2 * k].z, x0.z, acc, false);
        acc = __builtin_amdgcn_sdot4(R.c[2 * k].w, x0.w, acc, false);
        acc = __builtin_amdgcn_sdot4(R.c[2 * k + 1].x, x1.x, acc, false);
        acc = __builtin_amdgcn_sdot4(R.c[2 * k + 1].y, x1.y, acc, false);
        acc = __builtin_amdgcn_sdot4(R.c[2 * k + 1].z, x1.z, acc, false);
        acc = __builtin_amdgcn_sdot4(R.c[2 * k + 1].w, x1.w, acc, false);
        acc += dpp_i<DPP_QUAD_1032>(acc);
        t = ((float)acc * R.sc[k]) * S.xsc[0];
        if (CAP && half == 0) ((int32_t*)(a.capture + cap_offset(l, M_O) + cap_item(M_O).acc))[(size_t)i * H + h] = acc;
      }
      st_sc1(glb + i, pack(t, E));
    }
    if (wave == 1) dstamp(a.trace, l, 56);
    if (wave == 0) {
      xr = rs_o<Q8, CAP>(a, S, c, l, xr, bo);
      if (lane == 0) stamp(a.trace, 3 + 4 * l);
    }
    wg_barrier();  // the keys/values of block l are no longer read
    const int ln = l + 2;
    if (ln < L) {
      // int8: the next block's staging waits ~0.9 µs, past this block's reduce-scatter of
      // the output-projection terms (206.85 -> 206.4 µs; binary32 unchanged, so it does not)
      if constexpr (Q8) __builtin_amdgcn_s_sleep(32);
      load_o_head<Q8, H16>(R, (char*)&S.pr, a.w, ln, h);
      stage_kv(a, S, ln, h);
    }
    if (wave == 0) {
      if (ln < L) bo = small_p(a.w, ln, sp::B_O)[o];
      if (ln - 1 < L) bpr = small_p(a.w, ln - 1, sp::B_PR)[o];
    }
    wg_barrier();
  }
  if (!Q8 && c.set == 0) head_fill_wait();
  load_head_slots<Q8, H16>(R, a.w, head_rows_of<Q8>(c, wave));
  float x1p = 0.0f;
  if (c.set == 0) {
    if (wave == 0) x1p = x1_share(a, c, L - 1);
    rs_pr_poll<Q8>(a, S, c, L - 1, wave);
  }
  wg_barrier();
  if (wave == 0) {
    if (c.set == 0) rs_pr<Q8, CAP>(a, S, c, L - 1, bpr, x1p);
    gather<12>(loc_of(c, L - 1) + LO_X2, E, S.xs, hdr);
    if (lane == 0) stamp(a.trace, 49);
  }
}

// TR: the timestamp hook compiled in (it runs only when a.trace is set).  Without it
// the stores of the stamps, and the waits the compiler places after them, are gone.
template <bool Q8, bool CAP, bool TOKP, bool H16, bool TR>
__global__ __launch_bounds__(FT, 1) void k_fused(const FusedArgs a_in) {
  FusedArgs a = a_in;
  if constexpr (!TR) a.trace = nullptr;
  extern __shared__ __align__(16) char smem_raw[];
  FusedSmem& S = *(FusedSmem*)smem_raw;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  uint32_t* hdr = a.header;
  if (threadIdx.x == 0) stamp(a.trace, 0);
  Ctx c;
  c.E = ld32(&hdr[HDR_EPOCH]) + 1u;
  c.X = (int)xcc_id();
  const int rank = (int)blockIdx.x / NX;
  if (c.X >= NX) {
    if (threadIdx.x == 0) set_error(hdr, ERR_XCC);
    c.X = 0;
  }
  c.set = rank & 1;
  c.q = rank >> 1;
  c.nh = heads_of(c.X);
  c.head = c.q < c.nh;
  c.loc = a.fx + (size_t)c.X * L * FX_LOC_PER_LAYER;
  c.glb = a.fx + LOC_WORDS;
  float* sinkf = (float*)(a.sinkw + ((size_t)blockIdx.x * 8 + wave) * 16 + 8);
  const HeadRows hr = head_rows_of<Q8>(c, wave);  // this wave's head rows

  WRegs<Q8, H16> R;
  if (c.head) head_unit<Q8, CAP, TOKP, H16>(a, S, c, R, wave);
  else if (wave == 0) regular_io<Q8, CAP, TOKP, H16>(a, S, c, R);
  else regular_compute<Q8, CAP, H16>(a, S, c, R, wave);

  // ---- the tied head: every wave takes its head rows (the first ones are in its
  // registers already, except on the input wave of a regular unit of set 1, or of either
  // set for int8)
  if (!c.head && wave == 0 && (Q8 || c.set == 1)) load_head_slots<Q8, H16>(R, a.w, hr);
  wg_barrier();  // x12 is in LDS
  if constexpr (Q8) {
    layernorm_seq_wg<2>(S.xs, S.lnf[0], S.lnf[1], S.xn, S.lntmp, seq_tab(S), S.xc, S.xsc);
    wg_barrier();
    if (CAP && blockIdx.x == 0 && wave == 0) capture_input(a, S, 0, M_HEAD, S.xn, 0, D, lane, 64);
  }
  if (lane == 0 && wave == 1) stamp(a.trace, 55);
  head_rows<Q8, CAP, H16>(a, S, R, hr, sinkf);
  if (lane == 0 && wave == 1) stamp(a.trace, 50);

  // Epilogue: the last workgroup to finish checks the placement (XCD(b) - b one
  // constant mod NX, which the rank/XCD split above relies on; the waits would have
  // given up otherwise), then clears the counter and advances the epoch.
  __shared__ int s_last;
  __syncthreads();
  u64* place = a.fx + LOC_WORDS + GLB_WORDS;
  if (threadIdx.x == 0) {
    stamp(a.trace, 51);
    st_sc1(place + blockIdx.x, ((u64)c.E << 32) | (uint32_t)c.X);
    s_last = atomicAdd(&hdr[HDR_DONE], 1u) == (uint32_t)GRID - 1;
  }
  __syncthreads();
  if (s_last) {
    int bad = 0;
    if (threadIdx.x < GRID) {
      const int t = threadIdx.x;
      u64 w0, w;
      uint32_t spins = 0;
      do {
        w0 = ld_sc1(place);
        w = ld_sc1(place + t);
      } while ((epoch_of(w0) != c.E || epoch_of(w) != c.E) && ++spins < SPIN_LIMIT);
      const int off0 = ((int)(uint32_t)w0 + NX) % NX;
      const int off = ((int)(uint32_t)w - t % NX + NX) % NX;
      bad = off != off0 || epoch_of(w) != c.E || epoch_of(w0) != c.E;
    }
    bad = __syncthreads_or(bad);
    if (threadIdx.x == 0) {
      if (bad) set_error(hdr, ERR_XCC);
      // Every other workgroup has finished (and with it every wait that could set the
      // word), so a scratch shared by all calls can start the next launch clean.
      if (a.clear_error) {
        const uint32_t err = ld32(&hdr[HDR_ERROR]);
        if (a.status_out) *a.status_out = (int32_t)err;
        __hip_atomic_store(&hdr[HDR_ERROR], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      hdr[HDR_DONE] = 0;
      __hip_atomic_store(&hdr[HDR_EPOCH], c.E, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---- host side ---------------------------------------------------------------

struct FusedConfig {
  int ok;  // 1 usable, 0 not yet probed, -1 unusable (fall back to per-phase kernels)
};
static FusedConfig g_cfg[14][64];
uint64_t* g_fused_trace = nullptr;  // timeline test hook

template <bool Q8, bool CAP, bool TOKP, bool H16, bool TR>
static hipError_t fused_config(FusedConfig& c) {
  if (c.ok) return hipSuccess;
  int dev = 0, cus = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev))) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev))) return e;
  const size_t lds = sizeof(FusedSmem);
  if ((e = hipFuncSetAttribute((const void*)k_fused<Q8, CAP, TOKP, H16, TR>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)lds)))
    return e;
  int per_cu = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_fused<Q8, CAP, TOKP, H16, TR>, FT, lds))) return e;
  // One workgroup per compute unit, 32 per XCD: the grid is the whole chip.
  c.ok = (cus == GRID && per_cu >= 1) ? 1 : -1;
  return hipSuccess;
}

template <bool Q8, bool CAP, bool TOKP, bool H16, bool TR>
static hipError_t launch_fused_t(const Weights& w, const Work& k, uint32_t token, int32_t pos, float* cache,
                                 float* logits, char* capture, hipStream_t s, bool* used) {
  *used = false;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e) return e;
  FusedConfig& c = g_cfg[(H16 ? (TOKP ? 6 : 5) : TOKP ? (Q8 ? 4 : 3) : Q8 ? (CAP ? 2 : 1) : 0) + (TR ? 7 : 0)][dev & 63];
  if ((e = fused_config<Q8, CAP, TOKP, H16, TR>(c))) return e;
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
  a.status_out = k.step_status;
  a.clear_error = k.self_clearing ? 1u : 0u;
  a.token = token;
  a.pos = pos;
  // An ordinary launch of one workgroup per compute unit.  The waits between
  // workgroups need all 256 resident at once: fused_config admits the kernel only on
  // a device of exactly 256 compute units that fits one workgroup per unit (the LDS
  // size allows at most one), so on an otherwise idle GPU the dispatcher places all of
  // them at once.  If another kernel holds compute units (a GPU shared with other
  // work), a workgroup can wait for a unit that never frees: the waits then give up
  // after their bound, the error word is set and the step's outputs are invalid,
  // while the call itself has returned GPT2_OK.
  void* args[] = {&a};
  e = hipLaunchKernel((const void*)k_fused<Q8, CAP, TOKP, H16, TR>, dim3(GRID), dim3(FT), args, sizeof(FusedSmem), s);
  if (e == hipSuccess) *used = true;
  return e;
}

// The binary32 and binary16 steps run without the timestamp hook unless it is on.
// The int8 step keeps it compiled in: measured with and without it, the int8 kernel
// without the hook was slower (217.4 against 213.9 us), the binary32 one faster (128.6
// against 131.2 us).
template <bool Q8, bool CAP, bool TOKP, bool H16>
static hipError_t launch_fused_tr(const Weights& w, const Work& k, uint32_t token, int32_t pos, float* cache,
                                  float* logits, char* capture, hipStream_t s, bool* used) {
  if constexpr (Q8) {
    return launch_fused_t<Q8, CAP, TOKP, H16, true>(w, k, token, pos, cache, logits, capture, s, used);
  } else {
    if (g_fused_trace) return launch_fused_t<Q8, CAP, TOKP, H16, true>(w, k, token, pos, cache, logits, capture, s, used);
    return launch_fused_t<Q8, CAP, TOKP, H16, false>(w, k, token, pos, cache, logits, capture, s, used);
  }
}

hipError_t launch_fused(WFmt f, const Weights& w, const Work& k, uint32_t token, int32_t pos, float* cache,
                        float* logits, char* capture, hipStream_t s, bool* used, bool device_token) {
  if (capture && (f != WF_Q8 || device_token)) return hipErrorInvalidValue;
  if (f == WF_F16)
    return device_token ? launch_fused_tr<false, false, true, true>(w, k, token, pos, cache, logits, nullptr, s, used)
                        : launch_fused_tr<false, false, false, true>(w, k, token, pos, cache, logits, nullptr, s, used);
  const bool q8 = f == WF_Q8;
  if (device_token)
    return q8 ? launch_fused_tr<true, false, true, false>(w, k, token, pos, cache, logits, nullptr, s, used)
              : launch_fused_tr<false, false, true, false>(w, k, token, pos, cache, logits, nullptr, s, used);
  if (!q8) return launch_fused_tr<false, false, false, false>(w, k, token, pos, cache, logits, nullptr, s, used);
  if (capture) return launch_fused_tr<true, true, false, false>(w, k, token, pos, cache, logits, capture, s, used);
  return launch_fused_tr<true, false, false, false>(w, k, token, pos, cache, logits, nullptr, s, used);
}

}  // namespace g2
