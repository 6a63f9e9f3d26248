/* gpt2.h — GPT-2 124M single-token cached decode, full-prefix inference and the
 * int8 group-64 decode step on one AMD Instinct MI355X (gfx950).
 *
 * The model (LeanExe GPT-2 README, opening paragraph): 12 transformer blocks,
 * width 768, 12 heads, feed-forward width 3,072, a 50,257-token vocabulary,
 * binary32 arithmetic, weights supplied at run time.  Each block applies
 * LayerNorm, the query/key/value projection, causal attention, the output
 * projection with a residual add, LayerNorm and a tanh-GELU feed-forward network
 * with a residual add; a final LayerNorm and the shared token-embedding matrix
 * give the next-token logits.
 *
 * Conventions for every function below:
 *  - Device pointers are plain addresses of device memory that the CALLER owns
 *    (allocated by the caller, e.g. with torch); the library never allocates or
 *    frees device memory.  Device pointers must be 16-byte aligned, except the
 *    logits outputs, which need 4-byte alignment (rows of a [T][50257] array).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued on it
 *    and the call returns without waiting; GPT2_OK means "validated and
 *    enqueued".  A device fault would surface at the caller's next
 *    synchronisation.
 *  - Validation is done on the host from the scalar arguments only.  On any error
 *    the function returns a negative GPT2_E* code before enqueuing anything, and
 *    no output is written (the pages' entry points return empty arrays on invalid
 *    input).  Weight VALUES are never validated: non-finite binary32 weights are
 *    legal input and propagate (LeanExe README: the execution theorem covers every
 *    weight array of the right size, including exceptional values).
 *  - Calls that share a workspace or a cache must be ordered on one stream;
 *    concurrent streams need separate workspaces and caches.
 */
#ifndef GPT2_MI_H
#define GPT2_MI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Shape constants (LeanExe GPT-2 README, opening and checkpoint paragraphs). */
#define GPT2_LAYERS 12
#define GPT2_DMODEL 768
#define GPT2_HEADS 12
#define GPT2_DFF 3072
#define GPT2_VOCAB 50257
#define GPT2_MAX_POS 128              /* positions 0..127 are accepted */
#define GPT2_CKPT_WORDS 124439808u    /* packed checkpoint words ...   */
#define GPT2_CKPT_BYTES 497759232u    /* ... and bytes                 */
#define GPT2_CACHE_WORDS_PER_POS 18432 /* 12 layers x (768 keys + 768 values) */
#define GPT2_MAX_BATCH 64

enum {
  GPT2_PACK_F32 = 1, /* binary32 [out][in] matrices for the fp32 step, infer and the batched step */
  GPT2_PACK_Q8 = 2,  /* int8 group-64 codes and scales for gpt2_q8_cached_step */
  GPT2_PACK_F16 = 4  /* binary16 [out][in] block matrices and head for gpt2_f16_cached_step */
};

/* Stored weight format of a step (gpt2_generate's `weights`). */
enum { GPT2_WEIGHTS_F32 = 0, GPT2_WEIGHTS_Q8 = 1, GPT2_WEIGHTS_F16 = 2 };

enum {
  GPT2_OK = 0,
  GPT2_EWEIGHTS = -1,  /* checkpoint length is not 497,759,232 bytes, or null */
  GPT2_ETOKEN = -2,    /* token id >= 50,257, or a token array of length 0 or > 128 */
  GPT2_EPOSITION = -3, /* position outside 0..127 */
  GPT2_ECACHE = -4,    /* cache length != position * 18,432 words, or null cache */
  GPT2_ENOTPACKED = -5,/* the model was not packed in the form this call needs */
  GPT2_EARG = -6,      /* other invalid argument (null/misaligned pointer, short buffer, batch size) */
  GPT2_EHIP = -7       /* a HIP call failed while enqueuing */
};

typedef struct gpt2_model gpt2_model; /* opaque host handle */

/* Bytes of device memory the caller provides for the packed weights (flags: a
 * nonzero OR of GPT2_PACK_*).  0 for invalid flags. */
size_t gpt2_packed_nbytes(int flags);

/* Bytes of device workspace one stream needs (activations of up to 64 sessions,
 * the 128-row prefill buffers, the exchange buffers of the single-launch decode
 * step).  The caller zero-fills a workspace once before its first use; after that
 * the library keeps it consistent (its header holds a per-launch epoch).  Calls on
 * different streams need different workspaces. */
size_t gpt2_workspace_nbytes(void);

/* Re-lay the packed checkpoint for the device.
 *  ckpt_dev     : 124,439,808 little-endian binary32 words in the order of the
 *                 LeanExe README's checkpoint paragraph — token embeddings [50257][768],
 *                 all 1,024 position rows [1024][768], 12 blocks, final LayerNorm
 *                 gamma and beta.  Inside a block (GPT-2's own order, matrices
 *                 [input][output]): ln1 gamma, ln1 beta, qkv weight [768][2304] with
 *                 q|k|v columns, qkv bias, output-projection weight [768][768], its
 *                 bias, ln2 gamma, ln2 beta, fc weight [768][3072], fc bias,
 *                 mlp-projection weight [3072][768], its bias.
 *  ckpt_nbytes  : must be 497,759,232 (GPT2_EWEIGHTS otherwise).
 *  packed_dev   : >= gpt2_packed_nbytes(flags) bytes; written on `stream`.
 *  flags        : any nonzero OR of GPT2_PACK_F32, GPT2_PACK_Q8, GPT2_PACK_F16.  The
 *                 int8 form follows the marXiv 2609.00018 abstract: every block
 *                 matrix and the tied head, per output row and per group of 64
 *                 inputs, scale = max|w|/127, code = clamp(round-half-even(w/scale),
 *                 -127, 127).  The binary16 form (gpt2.s page, options, -h) rounds
 *                 the 48 block matrices and the head (the token table read as the
 *                 output matrix) to IEEE binary16, nearest with ties to even,
 *                 overflow to infinity; the embedding lookup keeps the binary32
 *                 table, which every form holds.
 *  out          : receives a host handle that refers to packed_dev (which must
 *                 stay allocated while the handle is used).  The checkpoint is
 *                 not referenced after the enqueued packing work completes.
 */
int gpt2_pack_weights(const void* ckpt_dev, size_t ckpt_nbytes, void* packed_dev, size_t packed_nbytes,
                      int flags, void* stream, gpt2_model** out);

/* gpt2_pack_weights with a chosen int8 weight-scale granularity (marXiv 2609.00018
 * abstract: its deployed model's 74.3 % smaller checkpoint matches one weight scale
 * per output row; its group-64 scales are the default).
 *  q8_weight_group : 64 (gpt2_pack_weights), 128, 192, 256, 384, 768, or 0 for one
 *                    scale per output row (768 inputs, 3,072 for the MLP projection).
 *                    Each output row's consecutive groups of that many inputs get
 *                    scale = max|w|/127 and codes clamp(round-half-even(w/scale),
 *                    -127, 127), 0 for an all-zero group.  The device form still
 *                    holds one scale per 64 inputs (the group's, repeated), so
 *                    every int8 entry point runs unchanged on it.
 * Other arguments and errors as gpt2_pack_weights; GPT2_EARG for another group. */
int gpt2_pack_weights_grouped(const void* ckpt_dev, size_t ckpt_nbytes, void* packed_dev, size_t packed_nbytes,
                              int flags, int q8_weight_group, void* stream, gpt2_model** out);

/* The int8 weight-scale group a model was packed with (0 = per row), -1 for null. */
int gpt2_q8_weight_group(const gpt2_model* model);

/* Free the host handle made by gpt2_pack_weights (the marXiv 2609.00018 abstract
 * lists buffer release among the obligations of a session).  The device memory
 * (packed weights, workspaces, caches) is the caller's and is not touched.  A null
 * handle is ignored; a handle must not be used after it is released. */
void gpt2_release(gpt2_model* model);

/* cachedStep (LeanExe GPT-2 README, cachedStep paragraph): one token at `position`.
 *  cache_dev    : caller's cache with room for (position+1)*18,432 words.  Its first
 *                 cache_nwords words are the incoming cache, ordered by prior position,
 *                 then layer, then 768 keys and 768 values: word
 *                 (source*12 + layer)*1536 + offset.  The step appends the current
 *                 position's 12 key/value rows in place (the returned cache is the
 *                 first (position+1)*18,432 words) and reads the supplied contents.
 *  cache_nwords : must equal position * 18,432 (GPT2_ECACHE otherwise).
 *  token        : 0..50,256.  position: 0..127.
 *  ws_dev       : gpt2_workspace_nbytes() bytes.
 *  logits_dev   : receives the 50,257 binary32 logits.
 * Needs a model packed with GPT2_PACK_F32. */
int gpt2_cached_step(const gpt2_model* model, float* cache_dev, size_t cache_nwords, uint32_t token,
                     int32_t position, void* ws_dev, float* logits_dev, void* stream);

/* The int8 group-64 cached step (marXiv 2609.00018 abstract): signed int8 weights
 * and projection inputs with one binary32 scale per 64 consecutive coordinates,
 * 32-bit integer group sums, binary32 everywhere else (embeddings, LayerNorm,
 * attention, GELU, residuals, the cache).  Each projection input is quantized per
 * group (scale = max|x|/127, code = clamp(round-half-even(x/scale), -127, 127)),
 * acc[j][g] = sum of 64 code products, and the output is
 * y = 0; y = y + ((float)acc[j][g] * wscale[j][g]) * xscale[g] for g = 0..G-1; y = y + bias.
 * Same arguments and errors as gpt2_cached_step; needs GPT2_PACK_Q8. */
int gpt2_q8_cached_step(const gpt2_model* model, float* cache_dev, size_t cache_nwords, uint32_t token,
                        int32_t position, void* ws_dev, float* logits_dev, void* stream);

/* The cached step with binary16 weight storage (gpt2.s page, options, -h): the 48
 * block matrices and the head are read as binary16 and widened exactly to binary32;
 * embeddings, biases, LayerNorm parameters, every product and sum, attention,
 * GELU, residuals and the cache stay binary32.  The result equals gpt2_cached_step
 * on a checkpoint whose block matrices and head were rounded to binary16 while the
 * embedding rows were not, bit for bit.  Same arguments and errors as
 * gpt2_cached_step; needs GPT2_PACK_F16. */
int gpt2_f16_cached_step(const gpt2_model* model, float* cache_dev, size_t cache_nwords, uint32_t token,
                         int32_t position, void* ws_dev, float* logits_dev, void* stream);

/* The int8 cached step with input scales per `input_group` consecutive coordinates
 * of each projection input (marXiv 2609.00018 abstract: its first design took one
 * scale per activation row, i.e. input_group = 0; its deployed one 64).
 *  input_group : 64, 128, 192, 256, 384, 768, or 0 for one scale per input vector.
 * With weight groups gw (gpt2_pack_weights_grouped) and input groups gx, the exact
 * int32 sums run over the gcd(gx, gw) consecutive coordinates on which both scales
 * are constant, and y = 0; y = y + ((float)acc_h * sw_h) * sx_h for those groups h
 * ascending; y = y + bias.  Scale and code rules as gpt2_q8_cached_step, which is
 * this call with input_group 64.  Input groups other than 64 run as one kernel per
 * phase.  Same arguments and errors as gpt2_cached_step, plus GPT2_EARG for another
 * group; needs GPT2_PACK_Q8. */
int gpt2_q8_cached_step_grouped(const gpt2_model* model, int input_group, float* cache_dev, size_t cache_nwords,
                                uint32_t token, int32_t position, void* ws_dev, float* logits_dev, void* stream);

/* B independent sessions (1..64) advanced by one token each: the cachedStep of the
 * LeanExe GPT-2 README applied to every session, with the batch invariance of the
 * muInference README's batch-invariance paragraph (a request's output does not
 * depend on what else is in the batch).
 *  caches_dev         : session b's cache starts at caches_dev + b*cache_stride_words;
 *                       same layout and in-place append as gpt2_cached_step.
 *  cache_stride_words : >= (max_b position[b] + 1) * 18,432 and a multiple of 4
 *                       (GPT2_ECACHE otherwise).  One allocation holds all B caches.
 *  cache_nwords_host, tokens_host, positions_host : host arrays of B entries, each
 *                       validated like gpt2_cached_step's scalars.
 *  B                  : 1..64 (GPT2_EARG otherwise).
 *  ws_dev             : gpt2_workspace_nbytes() bytes; it has room for 64 sessions.
 *  logits_dev         : [B][50,257].
 * Session b's logits and cache are bit-identical to gpt2_cached_step run on that
 * session alone.  Needs GPT2_PACK_F32. */
int gpt2_batched_cached_step(const gpt2_model* model, float* caches_dev, size_t cache_stride_words,
                             const size_t* cache_nwords_host, const uint32_t* tokens_host,
                             const int32_t* positions_host, int B, void* ws_dev, float* logits_dev,
                             void* stream);

/* gpt2_cached_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): no
 * workspace argument and no allocation of any kind.  The step's scratch (its header
 * and exchange area, GPT2_NOALLOC_SCRATCH_BYTES) is a static device array of the
 * library, one copy per GPU, held until the process ends; the first call on a GPU
 * looks up that GPU's copy.  Every call on one GPU shares it, so calls that overlap
 * on one GPU (several streams, several threads) race and give invalid results:
 * order them on one stream.  A batch-1 step needs a fixed amount of scratch, so no
 * input can exceed it; position is limited to 0..127 as for gpt2_cached_step.
 *  status_dev : device int32, or NULL.  Receives the step's error word (0 = fine,
 *               1 = a wait inside the step gave up, 2 = the workgroups were not
 *               dealt round-robin over the XCDs; then the logits are invalid).  The
 *               word is cleared after every call, so one failed call does not spoil
 *               the next.
 * The other arguments, the errors and the results are those of gpt2_cached_step
 * (same logits and cache, bit for bit).  The step must run as the single-launch
 * kernel (an MI355X with all 256 compute units free): GPT2_EHIP where it cannot. */
#define GPT2_NOALLOC_SCRATCH_BYTES 6555904u
int gpt2_cached_step_noalloc(const gpt2_model* model, float* cache_dev, size_t cache_nwords, uint32_t token,
                             int32_t position, float* logits_dev, int32_t* status_dev, void* stream);

/* infer (LeanExe GPT-2 README, infer paragraph): recompute a prefix of n = 1..128
 * tokens (host array; GPT2_ETOKEN for n outside 1..128 or any id >= 50,257) and
 * write the final row's 50,257 logits.  Needs GPT2_PACK_F32. */
int gpt2_infer(const gpt2_model* model, const uint32_t* tokens_host, int n, void* ws_dev, float* logits_dev,
               void* stream);

/* Error word of a workspace, given a host copy of at least its first 16 bytes:
 * 0 = fine; 1 = a wait inside the single-launch decode step gave up (after about
 * 2^21 polls); 2 = its workgroups were not dealt round-robin over the eight XCDs.
 * Either way that step's outputs, and those of every later step on the workspace,
 * are invalid (the waits of later steps return at once), and the word stays set
 * until the caller zero-fills the workspace again.  The single-launch step is one
 * ordinary launch of 256 workgroups, one per compute unit, whose waits need all of
 * them resident together: on a GPU that other work shares, a step can end this way
 * although the call returned GPT2_OK, so a caller that shares the GPU reads this
 * word after its steps. */
int gpt2_workspace_status(const void* ws_host_copy);

/* ---- test hooks (not needed by applications) -------------------------------- */

/* on != 0: gpt2_cached_step / gpt2_q8_cached_step use one kernel per block phase
 * instead of the single-launch step (same results; for testing both paths). */
void gpt2_test_force_phase_kernels(int on);

/* Timeline of the single-launch step: with trace_dev non-null (device buffer of
 * 256 x 64 uint64, row = workgroup), later steps write the device's 100 MHz
 * real-time counter per workgroup at its phase boundaries: slot 0 start; for
 * block l, on the units of the set that computes it, 1+4l the block input x in LDS
 * (head units: their share of the previous reduce-scatter done), 2+4l the unit's
 * QKV rows published (head units: attention output ready), 3+4l x1 in LDS (head
 * units: x1 share published), 4+4l the XCD's GELU slice in LDS (regular units);
 * 49 head input received, 55 head LayerNorm done, 50 head rows done, 51 end;
 * 52..63 finer points inside block 6.  Slots a unit does not reach are left as
 * they were.  The values computed are unchanged.  NULL turns it off. */
void gpt2_test_fused_trace(void* trace_dev);

/* Prefill that hands the session over to the cached step.  This is an extension:
 * the LeanExe README's infer returns logits only; the `lean` page's engine reuses
 * a prefix's cache.  It is gpt2_infer, plus the key/value rows of positions
 * 0..n-1 written into cache (device, at least n * 18,432 words) in the
 * cachedStep layout, so the session continues with gpt2_cached_step at position
 * n.  The rows are the ones the prefill's own attention used, so they are not
 * bit-identical to rows built by n cached steps (the sums are ordered
 * differently).  Errors: as gpt2_infer, and GPT2_ECACHE for a short or null
 * cache. */
int gpt2_prefill(const gpt2_model* model, const uint32_t* tokens, int n, float* cache_dev,
                 size_t cache_capacity_nwords, void* ws_dev, float* logits_dev, void* stream);

/* Greedy generation on the device.  The `lean` page's GPU path picks the next
 * token on the GPU, so a step never waits for the logits to reach the host; the
 * LeanExe README's command-line host generates a continuation greedily and rejects
 * non-finite logits.
 * Steps positions 0..n_prompt-1 with prompt (HOST array of n_prompt token ids),
 * then feeds each step the first maximum of the previous step's logits, until
 * n_gen tokens are chosen: tokens_out[i] (device, uint32[n_gen]) is the choice
 * made from the logits of position n_prompt-1+i, and the last choice is not
 * stepped, so positions 0..n_prompt+n_gen-2 are computed.  weights: GPT2_WEIGHTS_F32
 * (gpt2_cached_step, GPT2_PACK_F32), GPT2_WEIGHTS_Q8 (gpt2_q8_cached_step,
 * GPT2_PACK_Q8) or GPT2_WEIGHTS_F16 (gpt2_f16_cached_step, GPT2_PACK_F16).  cache (device) holds at
 * least (n_prompt+n_gen-1) * 18,432 words; it starts empty (position 0) and ends
 * holding those positions' rows.  logits receives the last step's logits.
 * *status (device int32) is 0 when every step's logits were finite, else k+1 for
 * the first step k (counted from the choice tokens_out[0]) whose logits held a
 * non-finite value: that choice and every later one are 50,257 (no token) and the
 * steps after it are fed token 0.  Everything is enqueued without host
 * synchronisation.  Errors: GPT2_ETOKEN for n_prompt < 1, n_gen < 1,
 * n_prompt+n_gen-1 > 128 or a prompt token >= 50,257; GPT2_ECACHE for a short or
 * null cache; GPT2_ENOTPACKED; GPT2_EARG otherwise. */
int gpt2_generate(const gpt2_model* model, float* cache_dev, size_t cache_capacity_nwords, const uint32_t* prompt,
                  int n_prompt, int n_gen, int weights, void* ws_dev, float* logits_dev, uint32_t* tokens_out_dev,
                  int32_t* status_dev, void* stream);

/* Group-64 quantizer alone: n (a multiple of 64) values -> codes [n], scales [n/64]. */
int gpt2_test_quantize(const float* x_dev, int n, int8_t* codes_dev, float* scales_dev, void* stream);

/* The int8 path's LayerNorm (ordered sums, one rounding per operation, gamma/beta
 * of 768 values), as the single-launch int8 step evaluates it with a whole
 * workgroup: rows x 768 values x -> y, bit for bit the ordered loop's result for
 * finite inputs.  rows 0 does nothing; rows < 0 is GPT2_EARG. */
int gpt2_test_layernorm_seq(const float* x_dev, int rows, const float* gamma_dev, const float* beta_dev,
                            float* y_dev, void* stream);

/* The library's exponential (kind 0) or tanh (kind 1) of every binary32 value whose
 * bit pattern is first_bits + i, i < n, into y[i].  The exponential is the ordered
 * binary32 approximation the decode path uses (LeanExe GPT-2 README, numerical
 * functions): k = rint(x*log2 e), Cody-Waite reduction r = (x - k*ln2_hi) - k*ln2_lo,
 * a degree-7 Taylor polynomial of e^r by Horner, times 2^k; x < -87 gives 0 and
 * x >= 88.72283935546875 gives +inf.  tanh(z) = 1 - 2/(exp(2|z|) + 1) with the sign of z. */
int gpt2_test_special(int kind, uint32_t first_bits, size_t n, float* y, void* stream);

/* C[M][N] = A[M][K] * W[N][K]^T with the prefill's split-K matrix-core kernel run
 * over all of K in one split (M 1..128, N a multiple of 32, K a multiple of 32). */
int gpt2_test_gemm(const float* A_dev, const float* W_dev, float* C_dev, int M, int N, int K, void* stream);

/* C[M][N] = A[M][K] * W[N][K]^T + bias[N], then tanh-GELU when gelu is 1, with the
 * prefill's full-K kernel of the MLP's first projection (M 1..128, N a multiple of 16,
 * K a multiple of 32; gelu 0 or 1). */
int gpt2_test_gemm_bias(const float* A_dev, const float* W_dev, const float* bias_dev, float* C_dev, int M, int N,
                        int K, int gelu, void* stream);

/* Bytes of the capture buffer of gpt2_q8_cached_step_capture. */
size_t gpt2_q8_capture_nbytes(void);

/* Byte offset inside the capture buffer of projection `matrix` (0 qkv, 1 output
 * projection, 2 fc, 3 mlp projection, 4 head) of `layer`, and of its parts:
 * input binary32 [K], input codes int8 [K], input scales [K/64], accumulators
 * int32 [N][K/64], output binary32 [N] (bias included, before residual/GELU). */
int gpt2_q8_capture_offsets(int layer, int matrix, size_t* base, size_t* in, size_t* codes, size_t* scales,
                            size_t* acc, size_t* out);

/* gpt2_q8_cached_step that also records every projection's operands (above). */
int gpt2_q8_cached_step_capture(const gpt2_model* model, float* cache_dev, size_t cache_nwords, uint32_t token,
                                int32_t position, void* ws_dev, float* logits_dev, void* capture_dev,
                                void* stream);

/* Device addresses of a packed matrix: matrix 0 qkv [2304][768], 1 output
 * projection [768][768], 2 fc [3072][768], 3 mlp projection [768][3072], 4 head
 * [50257][768] (layer ignored).  fp32 rows for GPT2_PACK_F32 (the head is the
 * token-embedding table), int8 codes and [rows][cols/64] scales for GPT2_PACK_Q8;
 * a pointer is null when that form was not packed. */
int gpt2_weight_view(const gpt2_model* model, int layer, int matrix, const float** f32_rows,
                     const int8_t** q8_codes, const float** q8_scales, int* rows, int* cols);

#ifdef __cplusplus
}
#endif
#endif
