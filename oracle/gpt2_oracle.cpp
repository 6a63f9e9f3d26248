// GPT-2 124M reference on the CPU — TEST INFRASTRUCTURE ONLY.
//
// Plain, slow, obviously correct definition of what the GPU library computes.
// Only the test-suite, the smoke check and the CPU-baseline leg of the bench load
// this library; the product path never does, and this file shares no code, header
// or table with the GPU library.
//
// Arithmetic: binary32 throughout (LeanExe GPT-2 README, opening paragraph: "binary32
// arithmetic"; every tensor word little-endian binary32).  Every sum runs
// sequentially in ascending index order; every product is rounded before it is
// added (built with -ffp-contract=off -fno-fast-math, the muInference page's "IEEE
// ops" table rule that FMA is not used where the source rounds twice).  Division
// and sqrtf are the correctly rounded IEEE operations.  The exponential is not the
// C library's: it is the ordered binary32 approximation defined below (exp_spec),
// and tanh is derived from it, so the whole forward pass is specified to the bit.
//
// Parity pins (see tests/test_oracle_*.py): closed-form sizes, the full-prefix ==
// cached recurrence identity, single-key attention == V exactly, softmax mass,
// library forward (transformers GPT-2 in float64) at tiny and full size, and
// hand-worked quantizer cases.  The end-to-end int8 logits are pinned only through
// their parts (quantizer cases, exact integer accumulators, a lossless-grid case
// and a float64 fake-quant forward); no page prints a logit value.
//
// OpenMP (optional) splits only independent output indices; every output keeps
// the same sequential sum, so the result is identical for any thread count.

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

extern "C" {

// Model shape.  GPT-2 124M: 12 blocks, width 768, 12 heads, feed-forward 3,072,
// vocabulary 50,257, 1,024 stored position rows, positions 0..127 accepted
// (LeanExe GPT-2 README, first and checkpoint paragraphs).
struct OracleDims {
  int32_t n_layer, d_model, n_head, d_ff, vocab, n_pos_rows, max_pos;
};

enum {
  ORACLE_OK = 0,
  ORACLE_EWEIGHTS = -1,
  ORACLE_ETOKEN = -2,
  ORACLE_EPOSITION = -3,
  ORACLE_ECACHE = -4,
  ORACLE_EARG = -6,
};

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"

namespace {

// ---- checkpoint layout ---------------------------------------------------
// Top-level order from the LeanExe README checkpoint paragraph: token embeddings,
// every stored position row, the blocks, the final normalisation.  Inside a block
// the page names only "block parameter offsets"; the reading taken here is GPT-2's
// own order with [input][output] matrices (gpt2.s page, weight-tiling paragraph).
enum Tensor {
  T_LN1_G = 0, T_LN1_B, T_ATTN_W, T_ATTN_B, T_APROJ_W, T_APROJ_B,
  T_LN2_G, T_LN2_B, T_FC_W, T_FC_B, T_MPROJ_W, T_MPROJ_B, T_BLOCK_COUNT
};

size_t block_tensor_words(const OracleDims& d, int t) {
  const size_t D = d.d_model, F = d.d_ff;
  switch (t) {
    case T_LN1_G: case T_LN1_B: case T_APROJ_B: case T_LN2_G: case T_LN2_B: case T_MPROJ_B:
      return D;
    case T_ATTN_W: return D * 3 * D;
    case T_ATTN_B: return 3 * D;
    case T_APROJ_W: return D * D;
    case T_FC_W: return D * F;
    case T_FC_B: return F;
    case T_MPROJ_W: return F * D;
  }
  return 0;
}

size_t block_words(const OracleDims& d) {
  size_t n = 0;
  for (int t = 0; t < T_BLOCK_COUNT; ++t) n += block_tensor_words(d, t);
  return n;
}

size_t wte_off(const OracleDims&) { return 0; }
size_t wpe_off(const OracleDims& d) { return (size_t)d.vocab * d.d_model; }
size_t block_off(const OracleDims& d, int layer) {
  return wpe_off(d) + (size_t)d.n_pos_rows * d.d_model + (size_t)layer * block_words(d);
}
size_t tensor_off(const OracleDims& d, int layer, int t) {
  size_t off = block_off(d, layer);
  for (int i = 0; i < t; ++i) off += block_tensor_words(d, i);
  return off;
}
size_t lnf_g_off(const OracleDims& d) { return block_off(d, d.n_layer); }
size_t lnf_b_off(const OracleDims& d) { return lnf_g_off(d) + d.d_model; }
size_t total_words(const OracleDims& d) { return lnf_b_off(d) + d.d_model; }

// Words in one cache row block: per prior position, per layer, D keys then D values
// (LeanExe README, cachedStep paragraph: index (source*12 + layer)*1536 + offset).
size_t cache_words_per_pos(const OracleDims& d) { return (size_t)d.n_layer * 2 * d.d_model; }

bool dims_ok(const OracleDims* d) {
  return d && d->n_layer > 0 && d->d_model > 0 && d->n_head > 0 && d->d_model % d->n_head == 0 &&
         d->d_ff > 0 && d->vocab > 0 && d->n_pos_rows > 0 && d->max_pos > 0 &&
         d->max_pos <= d->n_pos_rows && d->d_model % 64 == 0 && d->d_ff % 64 == 0;
}

// ---- numerical functions ---------------------------------------------------

// LayerNorm: mean, centred values, population variance, 1/sqrt(var + 1e-5),
// then (d*r)*gamma + beta.  The page says "normalization"; epsilon and the
// association are GPT-2's.
void layernorm(int n, const float* x, const float* g, const float* b, float* y) {
  float s = 0.0f;
  for (int i = 0; i < n; ++i) s = s + x[i];
  const float mu = s / (float)n;
  std::vector<float> dv(n);
  for (int i = 0; i < n; ++i) dv[i] = x[i] - mu;
  float v = 0.0f;
  for (int i = 0; i < n; ++i) v = v + dv[i] * dv[i];
  const float var = v / (float)n;
  const float r = 1.0f / std::sqrt(var + 1e-5f);
  for (int i = 0; i < n; ++i) y[i] = (dv[i] * r) * g[i] + b[i];
}

// Linear projection over the checkpoint's [in][out] layout:
// y_j = (sum_k x_k * W[k][j]) + b_j, the sum in ascending k.
void linear(int K, int N, const float* x, const float* W, const float* b, float* y) {
  const int JB = 256;
#pragma omp parallel for schedule(static)
  for (int j0 = 0; j0 < N; j0 += JB) {
    const int j1 = j0 + JB < N ? j0 + JB : N;
    float acc[JB];
    for (int j = j0; j < j1; ++j) acc[j - j0] = 0.0f;
    for (int k = 0; k < K; ++k) {
      const float xk = x[k];
      const float* row = W + (size_t)k * N;
      for (int j = j0; j < j1; ++j) acc[j - j0] = acc[j - j0] + xk * row[j];
    }
    for (int j = j0; j < j1; ++j) y[j] = b ? acc[j - j0] + b[j] : acc[j - j0];
  }
}

// ---- ordered binary32 exponential -------------------------------------------
// LeanExe GPT-2 README (source table, numerical functions) names an "ordered
// binary32 exponential approximation"; the muInference page (IEEE-ops table)
// builds exp from range reduction, a Taylor polynomial and 2^k assembled as a
// bit pattern, using only correctly rounded operations.  Definition used here,
// every step one rounded binary32 operation in this order:
//   x NaN -> x;  x >= 88.72283935546875 -> +inf;  x < -87 -> 0 (no subnormal results);
//   k = rint(x * log2(e));  r = (x - k*LN2_HI) - k*LN2_LO   (LN2_HI has 12 zero low bits,
//       so k*LN2_HI is exact);
//   p = 1/5040;  p = p*r + c for c = 1/720, 1/120, 1/24, 1/6, 1/2, 1, 1  (Horner, degree 7);
//   result = p * 2^k  (k = 128 is taken as (p*2) * 2^127).
float exp_spec(float x) {
  if (x != x) return x;
  if (x >= 88.72283935546875f) return INFINITY;
  if (x < -87.0f) return 0.0f;
  const float kf = std::rint(x * 1.44269502162933349609375f);
  const float LN2_HI = 0.693145751953125f;      // 0x3f317200
  const float LN2_LO = 1.428606765330187e-06f;  // ln 2 - LN2_HI
  const float r = (x - kf * LN2_HI) - kf * LN2_LO;
  float p = 1.0f / 5040.0f;
  p = p * r + 1.0f / 720.0f;
  p = p * r + 1.0f / 120.0f;
  p = p * r + 1.0f / 24.0f;
  p = p * r + 1.0f / 6.0f;
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  int k = (int)kf;
  if (k == 128) {
    p = p * 2.0f;
    k = 127;
  }
  uint32_t bits = (uint32_t)(k + 127) << 23;
  float scale;
  std::memcpy(&scale, &bits, 4);
  return p * scale;
}

// tanh from the exponential: t = 1 - 2/(exp(2|z|) + 1), sign of z restored.
float tanh_spec(float z) {
  const float e = exp_spec(2.0f * std::fabs(z));
  const float t = 1.0f - 2.0f / (e + 1.0f);
  return z < 0.0f ? -t : t;
}

// tanh form of GELU: 0.5*u*(1 + tanh(sqrt(2/pi)*(u + 0.044715*u^3))).
float gelu(float u) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi) rounded to binary32
  const float inner = u + 0.044715f * (u * u * u);
  const float t = tanh_spec(c * inner);
  return (0.5f * u) * (1.0f + t);
}

// One head of causal attention over npos keys.  Key j's dh coordinates start at
// kbase + j*stride, its values at vbase + j*stride.
//   s_j = (q . K_j) * (1/sqrt(dh));  m = max_j s_j;  e_j = exp(s_j - m);
//   Z = sum_j e_j;  w_j = e_j / Z;  a = sum_j w_j * V_j.
void attend_head(int dh, const float* q, const float* kbase, const float* vbase, size_t stride,
                 int npos, float* a, float* w_out) {
  const float scale = 1.0f / std::sqrt((float)dh);
  std::vector<float> s(npos), e(npos);
  for (int j = 0; j < npos; ++j) {
    const float* kj = kbase + (size_t)j * stride;
    float dot = 0.0f;
    for (int d = 0; d < dh; ++d) dot = dot + q[d] * kj[d];
    s[j] = dot * scale;
  }
  float m = s[0];
  for (int j = 1; j < npos; ++j)
    if (s[j] > m) m = s[j];
  float Z = 0.0f;
  for (int j = 0; j < npos; ++j) {
    e[j] = exp_spec(s[j] - m);
    Z = Z + e[j];
  }
  for (int j = 0; j < npos; ++j) e[j] = e[j] / Z;  // now the weights w_j
  for (int d = 0; d < dh; ++d) {
    float acc = 0.0f;
    for (int j = 0; j < npos; ++j) acc = acc + e[j] * vbase[(size_t)j * stride + d];
    a[d] = acc;
  }
  if (w_out)
    for (int j = 0; j < npos; ++j) w_out[j] = e[j];
}

// Tied vocabulary projection: logit_v = sum_i h_i * wte[v][i] (no bias).
void tied_logits(const OracleDims& d, const float* wte, const float* h, float* logits) {
  const int D = d.d_model;
#pragma omp parallel for schedule(static)
  for (int v = 0; v < d.vocab; ++v) {
    const float* row = wte + (size_t)v * D;
    float acc = 0.0f;
    for (int i = 0; i < D; ++i) acc = acc + h[i] * row[i];
    logits[v] = acc;
  }
}

// ---- int8 group-64 quantizer (marXiv 2609.00018 abstract) -------------------
// The abstract fixes scale selection, nearest-even rounding, saturation and the
// order of rescaling without printing formulas.  Reading taken: per group of 64
// consecutive coordinates, m = max|x|, s = m/127 (correctly rounded division);
// code = clamp(rint(x/s), -127, 127) with rint rounding half to even; a group
// with m == 0 gets s = 0 and all-zero codes.  NaN codes are 0.
int8_t code_of(float x, float s) {
  float q = std::rint(x / s);
  if (!(q == q)) q = 0.0f;
  if (q > 127.0f) q = 127.0f;
  if (q < -127.0f) q = -127.0f;
  return (int8_t)q;
}

void quant_group(const float* x, int n, int8_t* c, float* s_out) {
  float m = 0.0f;
  for (int i = 0; i < n; ++i) {
    const float a = std::fabs(x[i]);
    if (a > m) m = a;
  }
  if (m == 0.0f) {
    *s_out = 0.0f;
    for (int i = 0; i < n; ++i) c[i] = 0;
    return;
  }
  const float s = m / 127.0f;
  *s_out = s;
  for (int i = 0; i < n; ++i) c[i] = code_of(x[i], s);
}

// Quantized projection given quantized operands.  Row j has K codes wc[j][*] and
// K/64 group scales ws[j][*]; the input has codes xc and scales xs.
//   acc[j][g] = sum_{i<64} wc*xc  (exact int32)
//   y = 0;  for g ascending: y = y + ((float)acc * ws[j][g]) * xs[g];  y = y + b_j
void q8_linear_codes(int K, int N, const int8_t* xc, const float* xs, const int8_t* wc,
                     const float* ws, const float* b, int32_t* acc_out, float* y) {
  const int G = K / 64;
#pragma omp parallel for schedule(static)
  for (int j = 0; j < N; ++j) {
    const int8_t* row = wc + (size_t)j * K;
    float yj = 0.0f;
    for (int g = 0; g < G; ++g) {
      int32_t acc = 0;
      for (int i = 0; i < 64; ++i) acc += (int32_t)row[g * 64 + i] * (int32_t)xc[g * 64 + i];
      if (acc_out) acc_out[(size_t)j * G + g] = acc;
      yj = yj + ((float)acc * ws[(size_t)j * G + g]) * xs[g];
    }
    y[j] = b ? yj + b[j] : yj;
  }
}

void q8_linear(int K, int N, const float* x, const int8_t* wc, const float* ws, const float* b,
               float* y) {
  std::vector<int8_t> xc(K);
  std::vector<float> xs(K / 64);
  for (int g = 0; g < K / 64; ++g) quant_group(x + g * 64, 64, xc.data() + g * 64, &xs[g]);
  q8_linear_codes(K, N, xc.data(), xs.data(), wc, ws, b, nullptr, y);
}

// Oracle-side quantized weight store: per layer attn_w [3D][D], attnproj_w [D][D],
// fc_w [F][D], mlpproj_w [D][F] as [out][in] codes, then the head [V][D];
// scales [out][in/64] in the same order.
struct Q8Layout {
  size_t code_off[5], scale_off[5];  // per-layer matrices 0..3 relative to layer base; 4 = head
  size_t layer_codes, layer_scales, n_codes, n_scales;
};

Q8Layout q8_layout(const OracleDims& d) {
  Q8Layout q{};
  const size_t D = d.d_model, F = d.d_ff;
  const size_t rows[4] = {3 * D, D, F, D}, cols[4] = {D, D, D, F};
  size_t c = 0, s = 0;
  for (int m = 0; m < 4; ++m) {
    q.code_off[m] = c;
    q.scale_off[m] = s;
    c += rows[m] * cols[m];
    s += rows[m] * (cols[m] / 64);
  }
  q.layer_codes = c;
  q.layer_scales = s;
  q.code_off[4] = c * d.n_layer;
  q.scale_off[4] = s * d.n_layer;
  q.n_codes = q.code_off[4] + (size_t)d.vocab * D;
  q.n_scales = q.scale_off[4] + (size_t)d.vocab * (D / 64);
  return q;
}

// Quantize one checkpoint matrix stored [in][out] into [out][in] codes.
void quant_matrix_in_out(int K, int N, const float* W, int8_t* codes, float* scales) {
  const int G = K / 64;
#pragma omp parallel for schedule(static)
  for (int j = 0; j < N; ++j) {
    float col[64];
    for (int g = 0; g < G; ++g) {
      for (int i = 0; i < 64; ++i) col[i] = W[(size_t)(g * 64 + i) * N + j];
      quant_group(col, 64, codes + (size_t)j * K + g * 64, scales + (size_t)j * G + g);
    }
  }
}

// ---- quantizer granularity variants (marXiv 2609.00018 abstract) ------------
// The abstract's first design used one scale per activation row, its deployed one
// a scale per 64 consecutive coordinates, and its 74.3 % storage figure matches
// one weight scale per output row.  Generalised here: a weight scale per group of
// gw consecutive inputs of an output row and an input scale per group of gx
// consecutive coordinates, each group size a multiple of 64 dividing the row
// length K, or 0 for the whole row.  Scale choice, rounding and saturation are
// quant_group's.  The integer sums run over the groups on which both scales are
// constant (gcd(gx, gw) consecutive coordinates, since both partitions start at
// 0), and the rescale keeps the fixed order: y = 0; y = y + ((float)acc_h * sw) *
// sx for those groups h ascending; y = y + b.
int group_len(int g, int K) { return g == 0 ? K : g; }
bool group_ok(int g, int K) { return g == 0 || (g > 0 && g % 64 == 0 && K % g == 0); }
int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }

void qv_quantize_input(int K, const float* x, int gx, int8_t* xc, float* xs) {
  const int G = group_len(gx, K);
  for (int g = 0; g < K / G; ++g) quant_group(x + g * G, G, xc + g * G, &xs[g]);
}

// Row j: K codes wc[j][*] and K/gw scales ws[j][*]; the input: codes xc, K/gx scales xs.
void qv_linear_codes(int K, int N, const int8_t* xc, const float* xs, int gx, const int8_t* wc,
                     const float* ws, int gw, const float* b, int32_t* acc_out, float* y) {
  const int GX = group_len(gx, K), GW = group_len(gw, K), GM = gcd_int(GX, GW);
  const int NW = K / GW, NH = K / GM;
#pragma omp parallel for schedule(static)
  for (int j = 0; j < N; ++j) {
    const int8_t* row = wc + (size_t)j * K;
    float yj = 0.0f;
    for (int h = 0; h < NH; ++h) {
      int32_t acc = 0;
      for (int i = h * GM; i < (h + 1) * GM; ++i) acc += (int32_t)row[i] * (int32_t)xc[i];
      if (acc_out) acc_out[(size_t)j * NH + h] = acc;
      yj = yj + ((float)acc * ws[(size_t)j * NW + h * GM / GW]) * xs[h * GM / GX];
    }
    y[j] = b ? yj + b[j] : yj;
  }
}

// Oracle-side store of a variant: the Q8Layout order with K/gw scales per row.
Q8Layout qv_layout(const OracleDims& d, int gw) {
  Q8Layout q{};
  const size_t D = d.d_model, F = d.d_ff;
  const size_t rows[4] = {3 * D, D, F, D}, cols[4] = {D, D, D, F};
  size_t c = 0, s = 0;
  for (int m = 0; m < 4; ++m) {
    q.code_off[m] = c;
    q.scale_off[m] = s;
    c += rows[m] * cols[m];
    s += rows[m] * (cols[m] / group_len(gw, (int)cols[m]));
  }
  q.layer_codes = c;
  q.layer_scales = s;
  q.code_off[4] = c * d.n_layer;
  q.scale_off[4] = s * d.n_layer;
  q.n_codes = q.code_off[4] + (size_t)d.vocab * D;
  q.n_scales = q.scale_off[4] + (size_t)d.vocab * (D / group_len(gw, (int)D));
  return q;
}

int validate_step(const OracleDims* dm, size_t w_words, size_t cache_words, uint32_t tok,
                  int32_t pos) {
  if (!dims_ok(dm)) return ORACLE_EARG;
  const OracleDims& d = *dm;
  if (w_words != total_words(d)) return ORACLE_EWEIGHTS;
  if (tok >= (uint32_t)d.vocab) return ORACLE_ETOKEN;
  if (pos < 0 || pos >= d.max_pos) return ORACLE_EPOSITION;
  if (cache_words != (size_t)pos * cache_words_per_pos(d)) return ORACLE_ECACHE;
  return ORACLE_OK;
}

// ---- binary16 weight storage (gpt2.s page, options: -h) ----------------------
// The page keeps the 48 block matrices and the output head as half precision and
// everything else (embeddings, biases, LayerNorm weights, products, sums) in
// binary32.  It names no rounding rule for the conversion; the reading taken is
// IEEE 754's default, round to nearest with ties to even, overflow to infinity.
// binary16 has an 11-bit significand and exponents -14..15, so a finite nonzero x
// with floor(log2|x|) = e (at least -14) lies on the grid of spacing 2^(e-10);
// below 2^-14 the spacing stays 2^-24 (subnormals).  x / spacing is exact (a
// power-of-two scale), nearbyint rounds it to an integer with ties to even (the
// default rounding mode), and the product is exact again.
float round_binary16(float x) {
  if (!(x == x) || std::isinf(x) || x == 0.0f) return x;
  int e2 = 0;
  std::frexp(x, &e2);  // |x| = m 2^e2, 0.5 <= m < 1
  int e = e2 - 1;
  if (e < -14) e = -14;
  const float spacing = std::ldexp(1.0f, e - 10);
  const float r = std::nearbyint(x / spacing) * spacing;
  if (std::fabs(r) > 65504.0f) return std::copysign(INFINITY, x);
  return r;
}

// Per-projection hooks so the fp32 and the int8 forward share the block recurrence
// but not the projection arithmetic.
struct Proj {
  // matrix index m: 0 = attn_w, 1 = attnproj_w, 2 = fc_w, 3 = mlpproj_w, 4 = head
  virtual void run(int layer, int m, const float* x, float* y) const = 0;
  virtual ~Proj() {}
};

struct ProjF32 : Proj {
  const OracleDims& d;
  const float* w;
  ProjF32(const OracleDims& d_, const float* w_) : d(d_), w(w_) {}
  void run(int l, int m, const float* x, float* y) const override {
    const int D = d.d_model, F = d.d_ff;
    switch (m) {
      case 0: linear(D, 3 * D, x, w + tensor_off(d, l, T_ATTN_W), w + tensor_off(d, l, T_ATTN_B), y); break;
      case 1: linear(D, D, x, w + tensor_off(d, l, T_APROJ_W), w + tensor_off(d, l, T_APROJ_B), y); break;
      case 2: linear(D, F, x, w + tensor_off(d, l, T_FC_W), w + tensor_off(d, l, T_FC_B), y); break;
      case 3: linear(F, D, x, w + tensor_off(d, l, T_MPROJ_W), w + tensor_off(d, l, T_MPROJ_B), y); break;
      case 4: tied_logits(d, w + wte_off(d), x, y); break;
    }
  }
};

struct ProjQ8 : Proj {
  const OracleDims& d;
  const float* w;
  const int8_t* codes;
  const float* scales;
  Q8Layout q;
  ProjQ8(const OracleDims& d_, const float* w_, const int8_t* c_, const float* s_)
      : d(d_), w(w_), codes(c_), scales(s_), q(q8_layout(d_)) {}
  void run(int l, int m, const float* x, float* y) const override {
    const int D = d.d_model, F = d.d_ff;
    const int K[5] = {D, D, D, F, D}, N[5] = {3 * D, D, F, D, d.vocab};
    const int bt[4] = {T_ATTN_B, T_APROJ_B, T_FC_B, T_MPROJ_B};
    const size_t cb = m == 4 ? q.code_off[4] : l * q.layer_codes + q.code_off[m];
    const size_t sb = m == 4 ? q.scale_off[4] : l * q.layer_scales + q.scale_off[m];
    const float* b = m == 4 ? nullptr : w + tensor_off(d, l, bt[m]);
    q8_linear(K[m], N[m], x, codes + cb, scales + sb, b, y);
  }
};

struct ProjQv : Proj {
  const OracleDims& d;
  const float* w;
  const int8_t* codes;
  const float* scales;
  int gw, gx;
  Q8Layout q;
  ProjQv(const OracleDims& d_, const float* w_, const int8_t* c_, const float* s_, int gw_, int gx_)
      : d(d_), w(w_), codes(c_), scales(s_), gw(gw_), gx(gx_), q(qv_layout(d_, gw_)) {}
  void run(int l, int m, const float* x, float* y) const override {
    const int D = d.d_model, F = d.d_ff;
    const int K[5] = {D, D, D, F, D}, N[5] = {3 * D, D, F, D, d.vocab};
    const int bt[4] = {T_ATTN_B, T_APROJ_B, T_FC_B, T_MPROJ_B};
    const size_t cb = m == 4 ? q.code_off[4] : l * q.layer_codes + q.code_off[m];
    const size_t sb = m == 4 ? q.scale_off[4] : l * q.layer_scales + q.scale_off[m];
    const float* b = m == 4 ? nullptr : w + tensor_off(d, l, bt[m]);
    std::vector<int8_t> xc(K[m]);
    std::vector<float> xs(K[m] / group_len(gx, K[m]));
    qv_quantize_input(K[m], x, gx, xc.data(), xs.data());
    qv_linear_codes(K[m], N[m], xc.data(), xs.data(), gx, codes + cb, scales + sb, gw, b, nullptr, y);
  }
};

// One token through every block (LeanExe README: normalisation, QKV, causal
// attention, output projection + residual, normalisation, GELU feed-forward +
// residual; then final normalisation and the shared token-embedding matrix).
// The current key/value rows are appended to the cache first and attention reads
// every row 0..pos back from the cache at (source*L + layer)*2D + offset.
void step_body(const OracleDims& d, const float* w, const Proj& proj, float* cache, uint32_t tok,
               int32_t pos, float* logits) {
  const int D = d.d_model, F = d.d_ff, L = d.n_layer, H = d.n_head, dh = D / H;
  std::vector<float> x(D), h(D), qkv(3 * D), a(D), y(D), u(F);
  const float* wte = w + wte_off(d);
  const float* wpe = w + wpe_off(d);
  for (int i = 0; i < D; ++i) x[i] = wte[(size_t)tok * D + i] + wpe[(size_t)pos * D + i];
  const size_t rowstride = cache_words_per_pos(d);
  for (int l = 0; l < L; ++l) {
    layernorm(D, x.data(), w + tensor_off(d, l, T_LN1_G), w + tensor_off(d, l, T_LN1_B), h.data());
    proj.run(l, 0, h.data(), qkv.data());
    float* row = cache + ((size_t)pos * L + l) * 2 * D;
    for (int i = 0; i < D; ++i) {
      row[i] = qkv[D + i];
      row[D + i] = qkv[2 * D + i];
    }
    for (int hh = 0; hh < H; ++hh) {
      const float* kb = cache + (size_t)l * 2 * D + hh * dh;
      attend_head(dh, qkv.data() + hh * dh, kb, kb + D, rowstride, pos + 1, a.data() + hh * dh, nullptr);
    }
    proj.run(l, 1, a.data(), y.data());
    for (int i = 0; i < D; ++i) x[i] = x[i] + y[i];
    layernorm(D, x.data(), w + tensor_off(d, l, T_LN2_G), w + tensor_off(d, l, T_LN2_B), h.data());
    proj.run(l, 2, h.data(), u.data());
    for (int i = 0; i < F; ++i) u[i] = gelu(u[i]);
    proj.run(l, 3, u.data(), y.data());
    for (int i = 0; i < D; ++i) x[i] = x[i] + y[i];
  }
  layernorm(D, x.data(), w + lnf_g_off(d), w + lnf_b_off(d), h.data());
  proj.run(0, 4, h.data(), logits);
}

}  // namespace

extern "C" {

size_t oracle_ckpt_words(const OracleDims* d) { return dims_ok(d) ? total_words(*d) : 0; }

size_t oracle_cache_words_per_pos(const OracleDims* d) {
  return dims_ok(d) ? cache_words_per_pos(*d) : 0;
}

// Word offset of a tensor: tensor in 0..11 is the block tensor index (GPT-2 order),
// 100 = wte, 101 = wpe, 102 = lnf_g, 103 = lnf_b.
long long oracle_tensor_offset(const OracleDims* d, int layer, int tensor) {
  if (!dims_ok(d)) return -1;
  switch (tensor) {
    case 100: return (long long)wte_off(*d);
    case 101: return (long long)wpe_off(*d);
    case 102: return (long long)lnf_g_off(*d);
    case 103: return (long long)lnf_b_off(*d);
  }
  if (tensor < 0 || tensor >= T_BLOCK_COUNT || layer < 0 || layer >= d->n_layer) return -1;
  return (long long)tensor_off(*d, layer, tensor);
}

// cachedStep (LeanExe README, cachedStep paragraph).  cache holds cache_words =
// pos * L * 2D words on entry and must have room for (pos+1) * L * 2D; the current
// position's rows are appended.  logits receives vocab words.
int oracle_cached_step(const OracleDims* dm, const float* w, size_t w_words, float* cache,
                       size_t cache_words, uint32_t tok, int32_t pos, float* logits) {
  const int rc = validate_step(dm, w_words, cache_words, tok, pos);
  if (rc) return rc;
  ProjF32 p(*dm, w);
  step_body(*dm, w, p, cache, tok, pos, logits);
  return ORACLE_OK;
}

// infer (LeanExe README, infer paragraph): 1..max_pos tokens, the final row's
// logits.  Runs layer-major (all rows through block l before block l+1) with the
// keys and values kept in per-layer arrays instead of the cache, so its agreement
// with a chain of cachedStep calls checks the cache indexing and the recurrence.
int oracle_infer(const OracleDims* dm, const float* w, size_t w_words, const uint32_t* toks,
                 int n, float* logits) {
  if (!dims_ok(dm)) return ORACLE_EARG;
  const OracleDims& d = *dm;
  if (w_words != total_words(d)) return ORACLE_EWEIGHTS;
  if (n < 1 || n > d.max_pos || !toks) return ORACLE_ETOKEN;
  for (int t = 0; t < n; ++t)
    if (toks[t] >= (uint32_t)d.vocab) return ORACLE_ETOKEN;
  const int D = d.d_model, F = d.d_ff, H = d.n_head, dh = D / H;
  std::vector<float> X((size_t)n * D), Hn((size_t)n * D), QKV((size_t)n * 3 * D), A((size_t)n * D),
      Y(D), U(F);
  const float* wte = w + wte_off(d);
  const float* wpe = w + wpe_off(d);
  for (int t = 0; t < n; ++t)
    for (int i = 0; i < D; ++i)
      X[(size_t)t * D + i] = wte[(size_t)toks[t] * D + i] + wpe[(size_t)t * D + i];
  ProjF32 p(d, w);
  for (int l = 0; l < d.n_layer; ++l) {
    for (int t = 0; t < n; ++t) {
      layernorm(D, &X[(size_t)t * D], w + tensor_off(d, l, T_LN1_G), w + tensor_off(d, l, T_LN1_B),
                &Hn[(size_t)t * D]);
      p.run(l, 0, &Hn[(size_t)t * D], &QKV[(size_t)t * 3 * D]);
    }
    for (int t = 0; t < n; ++t)
      for (int hh = 0; hh < H; ++hh) {
        const float* kb = QKV.data() + D + hh * dh;
        attend_head(dh, &QKV[(size_t)t * 3 * D + hh * dh], kb, kb + D, 3 * (size_t)D, t + 1,
                    &A[(size_t)t * D + hh * dh], nullptr);
      }
    for (int t = 0; t < n; ++t) {
      p.run(l, 1, &A[(size_t)t * D], Y.data());
      for (int i = 0; i < D; ++i) X[(size_t)t * D + i] = X[(size_t)t * D + i] + Y[i];
      layernorm(D, &X[(size_t)t * D], w + tensor_off(d, l, T_LN2_G), w + tensor_off(d, l, T_LN2_B),
                &Hn[(size_t)t * D]);
      p.run(l, 2, &Hn[(size_t)t * D], U.data());
      for (int i = 0; i < F; ++i) U[i] = gelu(U[i]);
      p.run(l, 3, U.data(), Y.data());
      for (int i = 0; i < D; ++i) X[(size_t)t * D + i] = X[(size_t)t * D + i] + Y[i];
    }
  }
  layernorm(D, &X[(size_t)(n - 1) * D], w + lnf_g_off(d), w + lnf_b_off(d), Hn.data());
  tied_logits(d, wte, Hn.data(), logits);
  return ORACLE_OK;
}

// ---- int8 group-64 path (marXiv 2609.00018 abstract) -----------------------

void oracle_q8_sizes(const OracleDims* d, size_t* n_codes, size_t* n_scales) {
  if (!dims_ok(d)) {
    *n_codes = *n_scales = 0;
    return;
  }
  Q8Layout q = q8_layout(*d);
  *n_codes = q.n_codes;
  *n_scales = q.n_scales;
}

// Offsets (in elements) of matrix m (0 attn_w, 1 attnproj_w, 2 fc_w, 3 mlpproj_w,
// 4 head) of a layer in the oracle's own code and scale arrays.
void oracle_q8_offsets(const OracleDims* d, int layer, int m, size_t* code_off, size_t* scale_off) {
  Q8Layout q = q8_layout(*d);
  if (m == 4) {
    *code_off = q.code_off[4];
    *scale_off = q.scale_off[4];
  } else {
    *code_off = (size_t)layer * q.layer_codes + q.code_off[m];
    *scale_off = (size_t)layer * q.layer_scales + q.scale_off[m];
  }
}

// Weight quantization: every block matrix and the tied head, per output row, per
// group of 64 inputs.
int oracle_q8_quantize_weights(const OracleDims* dm, const float* w, size_t w_words, int8_t* codes,
                               float* scales) {
  if (!dims_ok(dm)) return ORACLE_EARG;
  const OracleDims& d = *dm;
  if (w_words != total_words(d)) return ORACLE_EWEIGHTS;
  const Q8Layout q = q8_layout(d);
  const int D = d.d_model, F = d.d_ff;
  const int wt[4] = {T_ATTN_W, T_APROJ_W, T_FC_W, T_MPROJ_W};
  const int K[4] = {D, D, D, F}, N[4] = {3 * D, D, F, D};
  for (int l = 0; l < d.n_layer; ++l)
    for (int m = 0; m < 4; ++m)
      quant_matrix_in_out(K[m], N[m], w + tensor_off(d, l, wt[m]),
                          codes + l * q.layer_codes + q.code_off[m],
                          scales + l * q.layer_scales + q.scale_off[m]);
  // head: wte rows are already [out][in]
  const float* wte = w + wte_off(d);
#pragma omp parallel for schedule(static)
  for (int v = 0; v < d.vocab; ++v)
    for (int g = 0; g < D / 64; ++g)
      quant_group(wte + (size_t)v * D + g * 64, 64, codes + q.code_off[4] + (size_t)v * D + g * 64,
                  scales + q.scale_off[4] + (size_t)v * (D / 64) + g);
  return ORACLE_OK;
}

// binary16 weight storage: a copy of the checkpoint whose 48 block matrices and
// token table are rounded to binary16 (round_binary16); every other word is copied
// unchanged.  The copy's token table is the rounded output head only: the step
// below still takes the embedding rows from the original checkpoint.
int oracle_f16_weights(const OracleDims* dm, const float* w, size_t w_words, float* w16) {
  if (!dims_ok(dm)) return ORACLE_EARG;
  const OracleDims& d = *dm;
  if (w_words != total_words(d)) return ORACLE_EWEIGHTS;
  std::memcpy(w16, w, w_words * sizeof(float));
  auto round_range = [&](size_t off, size_t n) {
    for (size_t i = 0; i < n; ++i) w16[off + i] = round_binary16(w[off + i]);
  };
  round_range(wte_off(d), (size_t)d.vocab * d.d_model);
  const int wt[4] = {T_ATTN_W, T_APROJ_W, T_FC_W, T_MPROJ_W};
  for (int l = 0; l < d.n_layer; ++l)
    for (int m = 0; m < 4; ++m) round_range(tensor_off(d, l, wt[m]), block_tensor_words(d, wt[m]));
  return ORACLE_OK;
}

// cachedStep with binary16 weight storage: the projections (block matrices and the
// head) read w16 from oracle_f16_weights, widened exactly to binary32, with the same
// binary32 arithmetic as oracle_cached_step; embeddings, LayerNorm and biases come
// from w.
int oracle_f16_cached_step(const OracleDims* dm, const float* w, const float* w16, size_t w_words, float* cache,
                           size_t cache_words, uint32_t tok, int32_t pos, float* logits) {
  const int rc = validate_step(dm, w_words, cache_words, tok, pos);
  if (rc) return rc;
  ProjF32 p(*dm, w16);
  step_body(*dm, w, p, cache, tok, pos, logits);
  return ORACLE_OK;
}

void oracle_round_binary16(long long n, const float* x, float* y) {
  for (long long i = 0; i < n; ++i) y[i] = round_binary16(x[i]);
}

// Quantized cachedStep: projections (the four block matrices and the tied head)
// take int8 weights and int8 inputs with group-64 scales; embeddings, LayerNorm,
// attention, GELU and residuals stay binary32 and are read from the fp32
// checkpoint.
int oracle_q8_cached_step(const OracleDims* dm, const float* w, size_t w_words,
                          const int8_t* codes, const float* scales, float* cache,
                          size_t cache_words, uint32_t tok, int32_t pos, float* logits) {
  const int rc = validate_step(dm, w_words, cache_words, tok, pos);
  if (rc) return rc;
  ProjQ8 p(*dm, w, codes, scales);
  step_body(*dm, w, p, cache, tok, pos, logits);
  return ORACLE_OK;
}

// Quantizer granularity variants (see qv_linear_codes).  Group sizes must be 0
// or multiples of 64 dividing both d_model and d_ff.
static bool qv_groups_ok(const OracleDims& d, int g) { return group_ok(g, d.d_model) && group_ok(g, d.d_ff); }

int oracle_qv_sizes(const OracleDims* d, int gw, size_t* n_codes, size_t* n_scales) {
  if (!dims_ok(d) || !qv_groups_ok(*d, gw)) return ORACLE_EARG;
  const Q8Layout q = qv_layout(*d, gw);
  *n_codes = q.n_codes;
  *n_scales = q.n_scales;
  return ORACLE_OK;
}

int oracle_qv_quantize_weights(const OracleDims* dm, const float* w, size_t w_words, int gw, int8_t* codes,
                               float* scales) {
  if (!dims_ok(dm) || !qv_groups_ok(*dm, gw)) return ORACLE_EARG;
  const OracleDims& d = *dm;
  if (w_words != total_words(d)) return ORACLE_EWEIGHTS;
  const Q8Layout q = qv_layout(d, gw);
  const int D = d.d_model, F = d.d_ff;
  const int wt[4] = {T_ATTN_W, T_APROJ_W, T_FC_W, T_MPROJ_W};
  const int K[4] = {D, D, D, F}, N[4] = {3 * D, D, F, D};
  for (int l = 0; l < d.n_layer; ++l)
    for (int m = 0; m < 4; ++m) {
      const float* W = w + tensor_off(d, l, wt[m]);  // [K][N]
      int8_t* c = codes + l * q.layer_codes + q.code_off[m];
      float* s = scales + l * q.layer_scales + q.scale_off[m];
      const int G = group_len(gw, K[m]), NG = K[m] / G;
#pragma omp parallel for schedule(static)
      for (int j = 0; j < N[m]; ++j) {
        std::vector<float> col(K[m]);
        for (int i = 0; i < K[m]; ++i) col[i] = W[(size_t)i * N[m] + j];
        for (int g = 0; g < NG; ++g)
          quant_group(col.data() + g * G, G, c + (size_t)j * K[m] + g * G, s + (size_t)j * NG + g);
      }
    }
  const float* wte = w + wte_off(d);
  const int G = group_len(gw, D), NG = D / G;
  for (int v = 0; v < d.vocab; ++v)
    for (int g = 0; g < NG; ++g)
      quant_group(wte + (size_t)v * D + g * G, G, codes + q.code_off[4] + (size_t)v * D + g * G,
                  scales + q.scale_off[4] + (size_t)v * NG + g);
  return ORACLE_OK;
}

int oracle_qv_cached_step(const OracleDims* dm, const float* w, size_t w_words, int gw, int gx,
                          const int8_t* codes, const float* scales, float* cache, size_t cache_words, uint32_t tok,
                          int32_t pos, float* logits) {
  if (!dims_ok(dm) || !qv_groups_ok(*dm, gw) || !qv_groups_ok(*dm, gx)) return ORACLE_EARG;
  const int rc = validate_step(dm, w_words, cache_words, tok, pos);
  if (rc) return rc;
  ProjQv p(*dm, w, codes, scales, gw, gx);
  step_body(*dm, w, p, cache, tok, pos, logits);
  return ORACLE_OK;
}

// One variant projection from binary32 input x: codes xc_out [K], input scales
// xs_out [K/gx], accumulators acc_out [N][K/gcd] (each optional), outputs y [N].
int oracle_qv_linear(int K, int N, const float* x, int gx, const int8_t* wc, const float* ws, int gw,
                     const float* b, int8_t* xc_out, float* xs_out, int32_t* acc_out, float* y) {
  if (K <= 0 || N < 0 || !group_ok(gx, K) || !group_ok(gw, K)) return ORACLE_EARG;
  std::vector<int8_t> xc(K);
  std::vector<float> xs(K / group_len(gx, K));
  qv_quantize_input(K, x, gx, xc.data(), xs.data());
  if (xc_out) std::memcpy(xc_out, xc.data(), K);
  if (xs_out) std::memcpy(xs_out, xs.data(), xs.size() * sizeof(float));
  qv_linear_codes(K, N, xc.data(), xs.data(), gx, wc, ws, gw, b, acc_out, y);
  return ORACLE_OK;
}

// ---- single operations, exposed for the brute-force and hand-case pins -----

void oracle_layernorm(int n, const float* x, const float* g, const float* b, float* y) {
  layernorm(n, x, g, b, y);
}

void oracle_linear(int K, int N, const float* x, const float* W_in_out, const float* b, float* y) {
  linear(K, N, x, W_in_out, b, y);
}

void oracle_gelu(int n, const float* x, float* y) {
  for (int i = 0; i < n; ++i) y[i] = gelu(x[i]);
}

// The specified exponential and tanh over n inputs (kind 0 = exp, 1 = tanh).
void oracle_special(int kind, long long n, const float* x, float* y) {
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < n; ++i) y[i] = kind == 0 ? exp_spec(x[i]) : tanh_spec(x[i]);
}

// Same over raw bit patterns [first, first + n): y[i] = f(bits_as_float(first + i)).
void oracle_special_bits(int kind, uint32_t first, long long n, float* y) {
#pragma omp parallel for schedule(static)
  for (long long i = 0; i < n; ++i) {
    const uint32_t b = first + (uint32_t)i;
    float x;
    std::memcpy(&x, &b, 4);
    y[i] = kind == 0 ? exp_spec(x) : tanh_spec(x);
  }
}

// q [dh]; K, V as [npos][stride] rows; a [dh]; w_out [npos] softmax weights.
void oracle_attention_head(int dh, const float* q, const float* K, const float* V, int stride,
                           int npos, float* a, float* w_out) {
  attend_head(dh, q, K, V, (size_t)stride, npos, a, w_out);
}

// Group-64 quantization of n values (n a multiple of 64).
int oracle_quantize(int n, const float* x, int8_t* codes, float* scales) {
  if (n < 0 || n % 64) return ORACLE_EARG;
  for (int g = 0; g < n / 64; ++g) quant_group(x + g * 64, 64, codes + g * 64, scales + g);
  return ORACLE_OK;
}

// Code rule with an explicit scale (rounding and saturation cases).
void oracle_quantize_with_scale(int n, const float* x, float s, int8_t* codes) {
  for (int i = 0; i < n; ++i) codes[i] = code_of(x[i], s);
}

// Quantized projection of an fp32 input: quantizes x per group, then the exact
// group accumulators and the fixed-order rescale.  Any of xc/xs/acc may be null.
int oracle_q8_linear(int K, int N, const float* x, const int8_t* wc, const float* ws,
                     const float* b, int8_t* xc_out, float* xs_out, int32_t* acc_out, float* y) {
  if (K <= 0 || K % 64 || N <= 0) return ORACLE_EARG;
  std::vector<int8_t> xc(K);
  std::vector<float> xs(K / 64);
  for (int g = 0; g < K / 64; ++g) quant_group(x + g * 64, 64, xc.data() + g * 64, &xs[g]);
  if (xc_out) std::memcpy(xc_out, xc.data(), K);
  if (xs_out) std::memcpy(xs_out, xs.data(), sizeof(float) * (K / 64));
  q8_linear_codes(K, N, xc.data(), xs.data(), wc, ws, b, acc_out, y);
  return ORACLE_OK;
}

// Same, from given input codes and scales.
void oracle_q8_linear_codes(int K, int N, const int8_t* xc, const float* xs, const int8_t* wc,
                            const float* ws, const float* b, int32_t* acc_out, float* y) {
  q8_linear_codes(K, N, xc, xs, wc, ws, b, acc_out, y);
}

}  // extern "C"
