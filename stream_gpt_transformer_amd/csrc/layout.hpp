// Model shape, packed-weight layout and workspace layout of the GPT-2 124M library.
// Shared by the host API and the kernels of this library (not by the CPU oracle).
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace g2 {

// GPT-2 124M (LeanExe GPT-2 README, opening and checkpoint paragraphs).
constexpr int D = 768;          // width
constexpr int H = 12;           // heads
constexpr int DH = 64;          // head width
constexpr int F = 3072;         // feed-forward width
constexpr int V = 50257;        // vocabulary
constexpr int L = 12;           // blocks
constexpr int PMAX = 128;       // positions accepted: 0..127
constexpr int NPOS_ROWS = 1024; // position rows stored in the checkpoint
constexpr int D3 = 3 * D;
constexpr int KV_ROW = 2 * D;            // words of one (position, layer) cache row: D keys, D values
constexpr int CACHE_POS = L * KV_ROW;    // 18,432 words per position
constexpr int MAX_BATCH = 64;

// ---- checkpoint (input) layout, in binary32 words --------------------------
// wte [V][D], wpe [1024][D], 12 blocks, lnf_g, lnf_b.  Inside a block (GPT-2's own
// order, [input][output] matrices): ln1_g, ln1_b, attn_w [D][3D], attn_b,
// attnproj_w [D][D], attnproj_b, ln2_g, ln2_b, fc_w [D][F], fc_b, mlpproj_w [F][D],
// mlpproj_b.
namespace ck {
constexpr size_t WTE = 0;
constexpr size_t WPE = (size_t)V * D;
constexpr size_t BLOCK0 = WPE + (size_t)NPOS_ROWS * D;
constexpr size_t LN1_G = 0, LN1_B = D, ATTN_W = 2 * D, ATTN_B = ATTN_W + (size_t)D * D3,
                 APROJ_W = ATTN_B + D3, APROJ_B = APROJ_W + (size_t)D * D, LN2_G = APROJ_B + D,
                 LN2_B = LN2_G + D, FC_W = LN2_B + D, FC_B = FC_W + (size_t)D * F,
                 MPROJ_W = FC_B + F, MPROJ_B = MPROJ_W + (size_t)F * D, BLOCK = MPROJ_B + D;
constexpr size_t LNF_G = BLOCK0 + (size_t)L * BLOCK;
constexpr size_t LNF_B = LNF_G + D;
constexpr size_t WORDS = LNF_B + D;
static_assert(BLOCK == 7087872, "block size");
static_assert(WORDS == 124439808, "checkpoint words");
}  // namespace ck

// ---- packed (device) layout, in bytes --------------------------------------
// Matrices are stored [out][in] row-major so a wavefront streams one output row
// with contiguous 16-byte loads.  The token-embedding table doubles as the tied
// head matrix (it is already [V][D]).
enum Mat { M_QKV = 0, M_O = 1, M_FC = 2, M_PR = 3, M_HEAD = 4 };
constexpr int mat_rows(int m) { return m == M_QKV ? D3 : m == M_FC ? F : m == M_HEAD ? V : D; }
constexpr int mat_cols(int m) { return m == M_PR ? F : D; }
constexpr size_t mat_elems(int m) { return (size_t)mat_rows(m) * mat_cols(m); }
constexpr size_t mat_elem_off(int m) {  // element offset of matrix m inside one layer
  return m == M_QKV ? 0 : m == M_O ? mat_elems(M_QKV) : m == M_FC ? mat_elems(M_QKV) + mat_elems(M_O)
                                                      : mat_elems(M_QKV) + mat_elems(M_O) + mat_elems(M_FC);
}
constexpr size_t LAYER_ELEMS = mat_elems(M_QKV) + mat_elems(M_O) + mat_elems(M_FC) + mat_elems(M_PR);
constexpr size_t mat_scale_off(int m) {  // group-scale offset of matrix m inside one layer
  return m == M_QKV ? 0 : m == M_O ? mat_elems(M_QKV) / 64 : m == M_FC ? (mat_elems(M_QKV) + mat_elems(M_O)) / 64
                                                         : (mat_elems(M_QKV) + mat_elems(M_O) + mat_elems(M_FC)) / 64;
}
constexpr size_t LAYER_SCALES = LAYER_ELEMS / 64;

// Small per-layer fp32 parameters, packed contiguously.
namespace sp {
constexpr int LN1_G = 0, LN1_B = D, B_QKV = 2 * D, B_O = B_QKV + D3, LN2_G = B_O + D, LN2_B = LN2_G + D,
              B_FC = LN2_B + D, B_PR = B_FC + F, PER_LAYER = B_PR + D;
constexpr int LNF_G = L * PER_LAYER, LNF_B = LNF_G + D, TOTAL = LNF_B + D;
}  // namespace sp

constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct PackedLayout {
  size_t wte, wpe, small, f32, q8_codes, q8_scales, f16, total;
};

// flags: bit 0 = fp32 matrices, bit 1 = int8 group-64 matrices, bit 2 = binary16
// matrices and token-embedding table.
constexpr int PACK_FLAGS_ALL = 7;
inline PackedLayout packed_layout(int flags) {
  PackedLayout p{};
  size_t off = 0;
  p.wte = off; off = align256(off + (size_t)V * D * 4);
  p.wpe = off; off = align256(off + (size_t)PMAX * D * 4);
  p.small = off; off = align256(off + (size_t)sp::TOTAL * 4);
  p.f32 = p.q8_codes = p.q8_scales = p.f16 = 0;
  if (flags & 1) { p.f32 = off; off = align256(off + (size_t)L * LAYER_ELEMS * 4); }
  if (flags & 2) {
    p.q8_codes = off; off = align256(off + (size_t)L * LAYER_ELEMS + (size_t)V * D);
    p.q8_scales = off; off = align256(off + ((size_t)L * LAYER_SCALES + (size_t)V * (D / 64)) * 4);
  }
  if (flags & 4) { p.f16 = off; off = align256(off + ((size_t)L * LAYER_ELEMS + (size_t)V * D) * 2); }
  p.total = off;
  return p;
}

// ---- workspace layout, in bytes --------------------------------------------
// header (uint32 words): [0] launch epoch of the fused step, [1] finished-workgroup
// counter, [2] error code (nonzero: a fused-step wait gave up).  A fresh workspace
// must be zero-filled.
struct WsLayout {
  size_t header, x, qkv, att, g, ll, pf_x, pf_h, pf_qkv, pf_att, pf_u, pf_part, total;
};

// Exchange area of the fused step, in 64-bit (epoch, value) words: per XCD and
// block the vectors exchanged inside the XCD (qkv of its heads 384 | attention
// output 128 | x1 768 | GELU slice 384 | x2 768), per block the partial terms of the
// two cross-XCD reductions (output projection 12 x 768 | MLP projection up to
// 48 x 768), one word per workgroup for the placement check, and one 128-byte line
// per wave (256 workgroups x 8 waves) that absorbs the stores of units it does not own.
constexpr int FX_NXCC = 8;
constexpr int FX_LOC_PER_LAYER = 384 + 128 + D + 384 + D;
constexpr int FX_GLB_PER_LAYER = (H + F / 64) * D;
constexpr size_t FX_WORDS = (size_t)FX_NXCC * L * FX_LOC_PER_LAYER + (size_t)L * FX_GLB_PER_LAYER + 256 + 256 * 8 * 16;
// Split-K partial sums of one prefill projection: at most S x 128 rows x N with
// S*N <= 12 * 768 (QKV 3 x 2304, O and MLP projection 8 x 768).
constexpr size_t PF_PART_WORDS = (size_t)12 * PMAX * D;

inline WsLayout ws_layout(int max_batch) {
  WsLayout w{};
  size_t off = 0;
  const size_t B = (size_t)(max_batch < 1 ? 1 : max_batch);
  w.header = off; off = align256(off + 256);
  w.x = off; off = align256(off + B * D * 4);
  w.qkv = off; off = align256(off + B * D3 * 4);
  w.att = off; off = align256(off + B * D * 4);
  w.g = off; off = align256(off + B * F * 4);
  w.ll = off; off = align256(off + FX_WORDS * 8);
  w.pf_x = off; off = align256(off + (size_t)PMAX * D * 4);
  w.pf_h = off; off = align256(off + (size_t)PMAX * D * 4);
  w.pf_qkv = off; off = align256(off + (size_t)PMAX * D3 * 4);
  w.pf_att = off; off = align256(off + (size_t)PMAX * D * 4);
  w.pf_u = off; off = align256(off + (size_t)PMAX * F * 4);
  w.pf_part = off; off = align256(off + PF_PART_WORDS * 4);
  w.total = off;
  return w;
}

// ---- int8 capture buffer (test hook), in bytes -------------------------------
// For each layer and projection m (0..3), then the head (m = 4):
//   input fp32 [K], codes int8 [K], input scales fp32 [K/64], accumulators int32
//   [N][K/64], output fp32 [N] (the projection value before any residual/GELU).
struct CapLayout {
  size_t in, codes, xs, acc, y, size;
};
constexpr CapLayout cap_item(int m) {
  const size_t K = mat_cols(m), N = mat_rows(m);
  CapLayout c{};
  size_t off = 0;
  c.in = off; off = align256(off + K * 4);
  c.codes = off; off = align256(off + K);
  c.xs = off; off = align256(off + K / 64 * 4);
  c.acc = off; off = align256(off + N * (K / 64) * 4);
  c.y = off; off = align256(off + N * 4);
  c.size = off;
  return c;
}
constexpr size_t cap_layer_bytes() {
  return cap_item(M_QKV).size + cap_item(M_O).size + cap_item(M_FC).size + cap_item(M_PR).size;
}
constexpr size_t cap_offset(int layer, int m) {
  if (m == M_HEAD) return (size_t)L * cap_layer_bytes();
  size_t off = (size_t)layer * cap_layer_bytes();
  for (int i = 0; i < m; ++i) off += cap_item(i).size;
  return off;
}
constexpr size_t cap_total() { return cap_offset(0, M_HEAD) + cap_item(M_HEAD).size; }

}  // namespace g2
