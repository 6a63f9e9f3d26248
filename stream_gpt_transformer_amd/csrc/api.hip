// C-ABI of the library: host-side validation, the model handle and dispatch to the
// kernel launchers.  Entry points and their input rules follow the LeanExe GPT-2
// README (infer and cachedStep paragraphs) and the marXiv 2609.00018 abstract.
#include <mutex>
#include <new>

#include "../../include/gpt2.h"
#include "internal.hpp"

using namespace g2;

struct gpt2_model {
  Weights w;
  int flags;
  int q8_group;  // int8 weight-scale group (coordinates; 0 = the whole row)
  const void* packed;
};

namespace g2 {
Work work_ptrs(void* ws, int max_batch) {
  const WsLayout l = ws_layout(max_batch);
  char* b = (char*)ws;
  Work k{};
  k.header = (uint32_t*)(b + l.header);
  k.x = (float*)(b + l.x);
  k.qkv = (float*)(b + l.qkv);
  k.att = (float*)(b + l.att);
  k.g = (float*)(b + l.g);
  k.ll = (unsigned long long*)(b + l.ll);
  k.pf_x = (float*)(b + l.pf_x);
  k.pf_h = (float*)(b + l.pf_h);
  k.pf_qkv = (float*)(b + l.pf_qkv);
  k.pf_att = (float*)(b + l.pf_att);
  k.pf_u = (float*)(b + l.pf_u);
  k.pf_part = (float*)(b + l.pf_part);
  return k;
}
}  // namespace g2

namespace g2 {
bool g_force_phase_kernels = false;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }
static bool aligned4(const void* p) { return ((uintptr_t)p & 3) == 0; }

static int step_checks(const gpt2_model* m, int need_flag, const float* cache, size_t cache_nwords,
                       uint32_t token, int32_t pos, const void* ws, const float* logits) {
  if (!m) return GPT2_EARG;
  if (!(m->flags & need_flag)) return GPT2_ENOTPACKED;
  if (token >= (uint32_t)V) return GPT2_ETOKEN;
  if (pos < 0 || pos >= PMAX) return GPT2_EPOSITION;
  if (!cache || !aligned16(cache) || cache_nwords != (size_t)pos * CACHE_POS) return GPT2_ECACHE;
  if (!ws || !aligned16(ws) || !logits || !aligned4(logits)) return GPT2_EARG;
  return GPT2_OK;
}

extern "C" {

size_t gpt2_packed_nbytes(int flags) {
  if (flags < 1 || flags > PACK_FLAGS_ALL) return 0;
  return packed_layout(flags).total;
}

size_t gpt2_workspace_nbytes(void) { return ws_layout(MAX_BATCH).total; }

// Scale-group sizes of the int8 granularity variants: 64, larger multiples of 64
// dividing 768 (so also 3,072), or 0 for the whole row.
static bool q8_group_ok(int g) { return g == 0 || (g > 0 && g % 64 == 0 && D % g == 0); }
static int q8_group_units(int g) { return g / 64; }  // 0 stays 0 (the whole row)

int gpt2_pack_weights(const void* ckpt_dev, size_t ckpt_nbytes, void* packed_dev, size_t packed_nbytes,
                      int flags, void* stream, gpt2_model** out) {
  return gpt2_pack_weights_grouped(ckpt_dev, ckpt_nbytes, packed_dev, packed_nbytes, flags, 64, stream, out);
}

int gpt2_pack_weights_grouped(const void* ckpt_dev, size_t ckpt_nbytes, void* packed_dev, size_t packed_nbytes,
                              int flags, int q8_weight_group, void* stream, gpt2_model** out) {
  if (!out || flags < 1 || flags > PACK_FLAGS_ALL || !q8_group_ok(q8_weight_group)) return GPT2_EARG;
  if (!ckpt_dev || ckpt_nbytes != (size_t)ck::WORDS * 4) return GPT2_EWEIGHTS;
  if (!aligned16(ckpt_dev)) return GPT2_EARG;
  if (!packed_dev || !aligned16(packed_dev) || packed_nbytes < packed_layout(flags).total) return GPT2_EARG;
  gpt2_model* m = new (std::nothrow) gpt2_model();
  if (!m) return GPT2_EARG;
  if (launch_pack((const float*)ckpt_dev, (char*)packed_dev, flags, (hipStream_t)stream, q8_weight_group) !=
      hipSuccess) {
    delete m;
    return GPT2_EHIP;
  }
  const PackedLayout pl = packed_layout(flags);
  const char* p = (const char*)packed_dev;
  m->flags = flags;
  m->q8_group = q8_weight_group;
  m->packed = packed_dev;
  m->w.wte = (const float*)(p + pl.wte);
  m->w.wpe = (const float*)(p + pl.wpe);
  m->w.small = (const float*)(p + pl.small);
  m->w.f32 = (flags & 1) ? (const float*)(p + pl.f32) : nullptr;
  m->w.q8c = (flags & 2) ? (const int8_t*)(p + pl.q8_codes) : nullptr;
  m->w.q8s = (flags & 2) ? (const float*)(p + pl.q8_scales) : nullptr;
  m->w.f16 = (flags & 4) ? (const uint16_t*)(p + pl.f16) : nullptr;
  *out = m;
  return GPT2_OK;
}

void gpt2_release(gpt2_model* model) { delete model; }

// One validated batch-1 step: the single-launch kernel, or the per-phase kernels
// where it cannot run.  tokp: read the token from device memory instead (it must be
// the workspace header's word HDR_WORD_NEXT_TOKEN).
// qx: the int8 input-scale group in units of 64 (0 = the whole row).  Only
// 64-coordinate input groups run in the single-launch kernel (which reads one
// weight scale per 64 inputs, replicated at packing for larger weight groups).
static int enqueue_step(const gpt2_model* m, WFmt f, float* cache, uint32_t token, const uint32_t* tokp,
                        int32_t pos, void* ws, float* logits, char* capture, hipStream_t s, int qx = 1) {
  const Work k = work_ptrs(ws, MAX_BATCH);
  bool used = false;
  if (!g_force_phase_kernels && qx == 1 &&
      launch_fused(f, m->w, k, token, pos, cache, logits, capture, s, &used, tokp != nullptr) != hipSuccess)
    return GPT2_EHIP;
  if (used) return GPT2_OK;
  Sessions ss{};
  ss.B = 1;
  ss.tok[0] = token;
  ss.pos[0] = pos;
  const hipError_t e = f == WF_Q8
                           ? launch_step_q8(m->w, k, ss, cache, logits, capture, s, tokp, qx, q8_group_units(m->q8_group))
                           : launch_step_f32(m->w, k, ss, cache, 0, logits, s, tokp, f == WF_F16);
  return e == hipSuccess ? GPT2_OK : GPT2_EHIP;
}

static int pack_flag(WFmt f) { return f == WF_Q8 ? GPT2_PACK_Q8 : f == WF_F16 ? GPT2_PACK_F16 : GPT2_PACK_F32; }

int gpt2_cached_step(const gpt2_model* m, float* cache, size_t cache_nwords, uint32_t token, int32_t pos,
                     void* ws, float* logits, void* stream) {
  const int rc = step_checks(m, GPT2_PACK_F32, cache, cache_nwords, token, pos, ws, logits);
  if (rc) return rc;
  return enqueue_step(m, WF_F32, cache, token, nullptr, pos, ws, logits, nullptr, (hipStream_t)stream);
}

int gpt2_f16_cached_step(const gpt2_model* m, float* cache, size_t cache_nwords, uint32_t token, int32_t pos,
                         void* ws, float* logits, void* stream) {
  const int rc = step_checks(m, GPT2_PACK_F16, cache, cache_nwords, token, pos, ws, logits);
  if (rc) return rc;
  return enqueue_step(m, WF_F16, cache, token, nullptr, pos, ws, logits, nullptr, (hipStream_t)stream);
}

static int q8_step(const gpt2_model* m, float* cache, size_t cache_nwords, uint32_t token, int32_t pos, void* ws,
                   float* logits, void* capture, void* stream) {
  const int rc = step_checks(m, GPT2_PACK_Q8, cache, cache_nwords, token, pos, ws, logits);
  if (rc) return rc;
  if (capture && !aligned16(capture)) return GPT2_EARG;
  return enqueue_step(m, WF_Q8, cache, token, nullptr, pos, ws, logits, (char*)capture, (hipStream_t)stream);
}

int gpt2_generate(const gpt2_model* m, float* cache, size_t cache_capacity_nwords, const uint32_t* prompt,
                  int n_prompt, int n_gen, int weights, void* ws, float* logits, uint32_t* tokens_out,
                  int32_t* status, void* stream) {
  if (!m || weights < GPT2_WEIGHTS_F32 || weights > GPT2_WEIGHTS_F16) return GPT2_EARG;
  const WFmt f = (WFmt)weights;
  if (!(m->flags & pack_flag(f))) return GPT2_ENOTPACKED;
  if (!prompt || n_prompt < 1 || n_gen < 1 || n_prompt + n_gen - 1 > PMAX) return GPT2_ETOKEN;
  for (int t = 0; t < n_prompt; ++t)
    if (prompt[t] >= (uint32_t)V) return GPT2_ETOKEN;
  const int nsteps = n_prompt + n_gen - 1;
  if (!cache || !aligned16(cache) || cache_capacity_nwords < (size_t)nsteps * CACHE_POS) return GPT2_ECACHE;
  if (!ws || !aligned16(ws) || !logits || !aligned4(logits) || !tokens_out || !aligned4(tokens_out) || !status ||
      !aligned4(status))
    return GPT2_EARG;
  const hipStream_t s = (hipStream_t)stream;
  uint32_t* next = work_ptrs(ws, MAX_BATCH).header + HDR_WORD_NEXT_TOKEN;
  for (int p = 0; p < nsteps; ++p) {
    const bool fed = p >= n_prompt;
    const int rc = enqueue_step(m, f, cache, fed ? 0u : prompt[p], fed ? next : nullptr, p, ws, logits, nullptr, s);
    if (rc) return rc;
    if (p >= n_prompt - 1 && launch_argmax(logits, next, tokens_out, status, p - (n_prompt - 1), s) != hipSuccess)
      return GPT2_EHIP;
  }
  return GPT2_OK;
}

int gpt2_q8_cached_step(const gpt2_model* m, float* cache, size_t cache_nwords, uint32_t token, int32_t pos,
                        void* ws, float* logits, void* stream) {
  return q8_step(m, cache, cache_nwords, token, pos, ws, logits, nullptr, stream);
}

int gpt2_q8_cached_step_grouped(const gpt2_model* m, int input_group, float* cache, size_t cache_nwords,
                                uint32_t token, int32_t pos, void* ws, float* logits, void* stream) {
  if (!q8_group_ok(input_group)) return GPT2_EARG;
  const int rc = step_checks(m, GPT2_PACK_Q8, cache, cache_nwords, token, pos, ws, logits);
  if (rc) return rc;
  return enqueue_step(m, WF_Q8, cache, token, nullptr, pos, ws, logits, nullptr, (hipStream_t)stream,
                      q8_group_units(input_group));
}

int gpt2_q8_weight_group(const gpt2_model* m) { return m ? m->q8_group : -1; }

// ---- gpt2_cached_step_noalloc: the batch-1 fp32 step without a caller workspace ----
// Its scratch is the single-launch step's header and exchange area, in a file-scope
// device array: each GPU the library runs on holds its own copy until the process
// ends.  In host code `scratch` names a host-side stand-in, not device memory, so the
// kernels get the address hipGetSymbolAddress returns for the current device.  The
// code-object loader zero-fills the array (an uninitialised ELF section), which is
// the state a fresh workspace must start in: epoch 0 in the header and in every
// exchange word.  After that each launch keeps it consistent by itself (the last
// workgroup resets the finished counter, advances the epoch and, here, reports and
// clears the error word), so no call clears anything.
}  // extern "C"
constexpr size_t NOALLOC_SCRATCH_BYTES = 256 + FX_WORDS * 8;  // header + exchange area, 6,555,904 B
static_assert(NOALLOC_SCRATCH_BYTES == GPT2_NOALLOC_SCRATCH_BYTES, "declared size");
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];
namespace {
constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[NOALLOC_MAX_DEVICES];

// The current device's copy of the scratch: looked up once per device, with that
// device current (the first call on it), then kept.
hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_noalloc_ptr[dev] = p;
  }
  *out = g_noalloc_ptr[dev];
  return hipSuccess;
}
}  // namespace
extern "C" {

int gpt2_cached_step_noalloc(const gpt2_model* m, float* cache, size_t cache_nwords, uint32_t token, int32_t pos,
                             float* logits, int32_t* status, void* stream) {
  if (!m) return GPT2_EARG;
  if (!(m->flags & GPT2_PACK_F32)) return GPT2_ENOTPACKED;
  if (token >= (uint32_t)V) return GPT2_ETOKEN;
  if (pos < 0 || pos >= PMAX) return GPT2_EPOSITION;
  if (!cache || !aligned16(cache) || cache_nwords != (size_t)pos * CACHE_POS) return GPT2_ECACHE;
  if (!logits || !aligned4(logits) || (status && !aligned4(status))) return GPT2_EARG;
  void* p = nullptr;
  if (noalloc_scratch(&p) != hipSuccess) return GPT2_EHIP;
  Work k{};
  k.header = (uint32_t*)p;
  k.ll = (unsigned long long*)((char*)p + 256);
  k.self_clearing = true;
  k.step_status = status;
  bool used = false;
  if (launch_fused(WF_F32, m->w, k, token, pos, cache, logits, nullptr, (hipStream_t)stream, &used) != hipSuccess)
    return GPT2_EHIP;
  return used ? GPT2_OK : GPT2_EHIP;
}

int gpt2_q8_cached_step_capture(const gpt2_model* m, float* cache, size_t cache_nwords, uint32_t token,
                                int32_t pos, void* ws, float* logits, void* capture, void* stream) {
  if (!capture) return GPT2_EARG;
  return q8_step(m, cache, cache_nwords, token, pos, ws, logits, capture, stream);
}

int gpt2_batched_cached_step(const gpt2_model* m, float* caches, size_t stride, const size_t* cache_nwords,
                             const uint32_t* tokens, const int32_t* positions, int B, void* ws, float* logits,
                             void* stream) {
  if (!m) return GPT2_EARG;
  if (!(m->flags & GPT2_PACK_F32)) return GPT2_ENOTPACKED;
  if (B < 1 || B > MAX_BATCH || !cache_nwords || !tokens || !positions) return GPT2_EARG;
  if (!ws || !aligned16(ws) || !logits || !aligned4(logits)) return GPT2_EARG;
  if (!caches || !aligned16(caches) || (stride & 3)) return GPT2_ECACHE;
  Sessions ss{};
  ss.B = B;
  for (int b = 0; b < B; ++b) {
    if (tokens[b] >= (uint32_t)V) return GPT2_ETOKEN;
    if (positions[b] < 0 || positions[b] >= PMAX) return GPT2_EPOSITION;
    if (cache_nwords[b] != (size_t)positions[b] * CACHE_POS) return GPT2_ECACHE;
    if (stride < (size_t)(positions[b] + 1) * CACHE_POS) return GPT2_ECACHE;
    ss.tok[b] = tokens[b];
    ss.pos[b] = positions[b];
  }
  const hipError_t e =
      launch_step_f32(m->w, work_ptrs(ws, MAX_BATCH), ss, caches, stride, logits, (hipStream_t)stream);
  return e == hipSuccess ? GPT2_OK : GPT2_EHIP;
}

int gpt2_prefill(const gpt2_model* m, const uint32_t* tokens, int n, float* cache, size_t cache_capacity_nwords,
                 void* ws, float* logits, void* stream) {
  if (!m) return GPT2_EARG;
  if (!(m->flags & GPT2_PACK_F32)) return GPT2_ENOTPACKED;
  if (!tokens || n < 1 || n > PMAX) return GPT2_ETOKEN;
  for (int t = 0; t < n; ++t)
    if (tokens[t] >= (uint32_t)V) return GPT2_ETOKEN;
  if (!cache || !aligned16(cache) || cache_capacity_nwords < (size_t)n * CACHE_POS) return GPT2_ECACHE;
  if (!ws || !aligned16(ws) || !logits || !aligned4(logits)) return GPT2_EARG;
  const hipError_t e = launch_infer(m->w, work_ptrs(ws, MAX_BATCH), tokens, n, logits, (hipStream_t)stream, cache);
  return e == hipSuccess ? GPT2_OK : GPT2_EHIP;
}

int gpt2_infer(const gpt2_model* m, const uint32_t* tokens, int n, void* ws, float* logits, void* stream) {
  if (!m) return GPT2_EARG;
  if (!(m->flags & GPT2_PACK_F32)) return GPT2_ENOTPACKED;
  if (!tokens || n < 1 || n > PMAX) return GPT2_ETOKEN;
  for (int t = 0; t < n; ++t)
    if (tokens[t] >= (uint32_t)V) return GPT2_ETOKEN;
  if (!ws || !aligned16(ws) || !logits || !aligned4(logits)) return GPT2_EARG;
  const hipError_t e = launch_infer(m->w, work_ptrs(ws, MAX_BATCH), tokens, n, logits, (hipStream_t)stream);
  return e == hipSuccess ? GPT2_OK : GPT2_EHIP;
}

int gpt2_test_quantize(const float* x, int n, int8_t* codes, float* scales, void* stream) {
  if (n < 0 || n % 64 || (n && (!x || !codes || !scales))) return GPT2_EARG;
  return launch_quantize(x, n, codes, scales, (hipStream_t)stream) == hipSuccess ? GPT2_OK : GPT2_EHIP;
}

int gpt2_test_layernorm_seq(const float* x, int rows, const float* gamma, const float* beta, float* y,
                            void* stream) {
  if (rows < 0 || (rows && (!x || !gamma || !beta || !y))) return GPT2_EARG;
  return launch_layernorm_seq(x, rows, gamma, beta, y, (hipStream_t)stream) == hipSuccess ? GPT2_OK : GPT2_EHIP;
}

int gpt2_test_special(int kind, uint32_t first_bits, size_t n, float* y, void* stream) {
  if ((kind != 0 && kind != 1) || n > ((size_t)1 << 32) - first_bits || (n && !y)) return GPT2_EARG;
  return launch_special_bits(kind, first_bits, (long long)n, y, (hipStream_t)stream) == hipSuccess ? GPT2_OK : GPT2_EHIP;
}

int gpt2_test_gemm(const float* A, const float* W, float* C, int M, int N, int K, void* stream) {
  if (!A || !W || !C || M < 1 || M > PMAX || N < 32 || N % 32 || K < 32 || K % 32) return GPT2_EARG;
  return launch_gemm_test(A, W, C, M, N, K, (hipStream_t)stream) == hipSuccess ? GPT2_OK : GPT2_EHIP;
}

int gpt2_test_gemm_bias(const float* A, const float* W, const float* bias, float* C, int M, int N, int K, int gelu,
                        void* stream) {
  if (!A || !W || !bias || !C || M < 1 || M > PMAX || N < 16 || N % 16 || K < 32 || K % 32 || (gelu != 0 && gelu != 1))
    return GPT2_EARG;
  return launch_gemm16_test(A, W, bias, C, M, N, K, gelu != 0, (hipStream_t)stream) == hipSuccess ? GPT2_OK : GPT2_EHIP;
}

void gpt2_test_force_phase_kernels(int on) { g_force_phase_kernels = on != 0; }

void gpt2_test_fused_trace(void* trace_dev) { g_fused_trace = (uint64_t*)trace_dev; }

int gpt2_workspace_status(const void* ws_host_copy) {
  return ws_host_copy ? (int)((const uint32_t*)ws_host_copy)[2] : 0;
}

size_t gpt2_q8_capture_nbytes(void) { return cap_total(); }

int gpt2_q8_capture_offsets(int layer, int matrix, size_t* base, size_t* in, size_t* codes, size_t* scales,
                            size_t* acc, size_t* out) {
  if (matrix < 0 || matrix > 4 || (matrix < 4 && (layer < 0 || layer >= L))) return GPT2_EARG;
  const CapLayout c = cap_item(matrix);
  const size_t b = cap_offset(matrix == 4 ? 0 : layer, matrix);
  if (base) *base = b;
  if (in) *in = b + c.in;
  if (codes) *codes = b + c.codes;
  if (scales) *scales = b + c.xs;
  if (acc) *acc = b + c.acc;
  if (out) *out = b + c.y;
  return GPT2_OK;
}

int gpt2_weight_view(const gpt2_model* m, int layer, int matrix, const float** f32_rows, const int8_t** codes,
                     const float** scales, int* rows, int* cols) {
  if (!m || matrix < 0 || matrix > 4 || (matrix < 4 && (layer < 0 || layer >= L))) return GPT2_EARG;
  if (rows) *rows = mat_rows(matrix);
  if (cols) *cols = mat_cols(matrix);
  if (f32_rows) *f32_rows = matrix == 4 ? m->w.wte : (m->w.f32 ? f32_mat(m->w, layer, matrix) : nullptr);
  if (codes) *codes = m->w.q8c ? q8_codes(m->w, layer, matrix) : nullptr;
  if (scales) *scales = m->w.q8s ? q8_scales(m->w, layer, matrix) : nullptr;
  return GPT2_OK;
}

}  // extern "C"
