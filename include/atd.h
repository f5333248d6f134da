/*
 * atd.h -- C ABI of the MI355X (gfx950) decode-step library.
 *
 * The library runs the autoregressive decode step of a Qwen-style decoder
 * stack on one GPU: input embedding sum, per layer RMSNorm + q/k/v
 * projection, per-head QK RMSNorm + RoPE + KV-cache append, causal GQA
 * attention over the cache, output projection + residual, RMSNorm + SwiGLU
 * MLP + residual, then the final RMSNorm and an LM head; plus penalized
 * greedy argmax and KV bucket growth.
 *
 * Sources (page title, section):
 *  - "Qwen3-TTS ncnn port" (ncnn discussion 6799), "Talker: non-standard
 *    structure and two-level generation": QK RMSNorm over head_dim after
 *    the q/k projections, 8 KV heads shared by 16 query heads, interleaved
 *    mRoPE equal to plain RoPE for TTS, the frame loop, repetition penalty.
 *  - "Audio8-ASR dynamic KV-cache bucket" (RK3576 acceptance report),
 *    "dynamic window mechanism": external [heads, Smax, head_dim] cache
 *    owned and written by the host side, growth by copying the valid region
 *    to a larger buffer and continuing at the same token and RoPE position,
 *    no sliding window.
 *  - "qwen3-tts-hip OPTIMIZATION_LOG", DecodeStepStack profile entry (the
 *    per-layer sequence of operations) and the repetition-penalty entry.
 *  - "NEON library" maintainers page, "Contracts": input storage stays valid
 *    during a call, outputs belong to the caller, validation happens before
 *    any work starts and leaves the object reusable, one object is used
 *    serially.
 *
 * Conventions for every entry point:
 *  - Pointers documented as "device" are HIP device memory of the current
 *    device, owned by the caller; "host" pointers are read during the call
 *    only.  Weights and KV buffers must stay allocated while a decoder that
 *    references them is in use.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously on it; outputs are valid once the stream reaches that
 *    point.  Results never depend on the stream.
 *  - Every argument is checked on the host before anything is enqueued.  On
 *    any error other than ATD_ERR_DEVICE nothing was enqueued and the decoder
 *    is unchanged and reusable.  decoder_last_error() names the refused
 *    argument and its value.  There is no fallback path: an unsupported
 *    configuration is an error.
 *  - All floating-point activations, hidden states, logits and biases are
 *    float32.  Weights and embedding tables are stored in atd_config.dtype,
 *    the KV cache in atd_config.kv_dtype (float32 or bf16 each); arithmetic
 *    accumulates in float32.
 *  - A decoder is used from one host thread at a time.
 *  - With the environment variable ATD_ROCTX=1, each entry point's enqueue
 *    (and each layer of a step) is wrapped in a ROCTx range named after it,
 *    for timelines (rocprofv3 --marker-trace); off otherwise.
 */
#ifndef ATD_H
#define ATD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  ATD_OK = 0,
  ATD_ERR_INVALID_ARG = -1, /* null/misaligned pointer, value out of range   */
  ATD_ERR_SHAPE = -2,       /* sizes inconsistent with the config           */
  ATD_ERR_DTYPE = -3,       /* unknown storage dtype                        */
  ATD_ERR_KV_FULL = -4,     /* the write position reached the KV capacity   */
  ATD_ERR_CAPACITY = -5,    /* beyond max_rows / max_slots / max_ctx, or a
                               bucket too small for the valid rows           */
  ATD_ERR_DEVICE = -6,      /* a HIP call failed (message names the error)  */
  ATD_ERR_UNSUPPORTED = -7  /* config outside what the kernels implement    */
};

/* Storage dtypes of weights and embedding tables (atd_config.dtype) and of
 * the KV cache (atd_config.kv_dtype). */
enum { ATD_F32 = 0, ATD_BF16 = 1 };

/* Shape of one decoder stack (hyper-parameters; host struct). */
typedef struct atd_config {
  int32_t n_layers;    /* L >= 1                                             */
  int32_t hidden;      /* h, multiple of 8, <= 8192 (<= 4096 for F32)       */
  int32_t n_q_heads;   /* Hq                                                 */
  int32_t n_kv_heads;  /* Hkv; Hq / Hkv in {1, 2, 4, 8}                      */
  int32_t head_dim;    /* D in {64, 128}                                     */
  int32_t ffn;         /* F, multiple of 8, <= 8192 (<= 4096 for F32)       */
  int32_t vocab;       /* V of every LM head, >= 2                           */
  int32_t n_lm_heads;  /* number of LM heads (15 for the code predictor)     */
  int32_t n_tables;    /* number of embedding tables, 1..16                  */
  int32_t qk_norm;     /* 1: per-head RMSNorm of q and k before RoPE         */
  int32_t qkv_bias;    /* 1: q/k/v projections carry a bias                  */
  int32_t dtype;       /* weights and embedding tables: ATD_F32 or ATD_BF16  */
  int32_t kv_dtype;    /* KV cache rows: ATD_F32 or ATD_BF16 (rounded to
                          nearest even when stored)                         */
  double rope_theta;   /* RoPE base (1e6 for the Qwen3 Talker)               */
  float rms_eps;       /* epsilon of every RMSNorm                           */
  int32_t max_slots;   /* independent streams (KV caches) the decoder keeps  */
  int32_t max_rows;    /* largest B of a step / T of a prefill               */
  int32_t max_ctx;     /* largest number of cached rows any slot reaches     */
  int32_t flags;       /* ATD_FLAG_* bits                                    */
  int32_t weight_format; /* ATD_WFMT_*: storage of the seven per-layer
                            matrices (LM heads and tables stay in dtype)     */
  int32_t input_dim;   /* width of the input rows (tables, extra, prefill
                          rows): 0 or hidden, or another multiple of 8 <=
                          8192 (<= 4096 for F32) with an input projection   */
  int32_t mrope_sections[3]; /* (s_t, s_h, s_w) frequency counts of the
                          interleaved multimodal RoPE used by the *_mrope
                          entry points; {0, 0, 0}: every frequency follows
                          the t position.  See decoder_prefill_mrope.      */
} atd_config;

/* atd_config.weight_format ("Rockchip NPU sidecars" page, section "The talker
 * is the only DRAM-bound candidate": the Talker's matmuls as Q8_0, 32 int8
 * weights and one fp16 scale per block, and re-quantized to Q4_K at 47%
 * fewer bytes).  Quantized matrices keep their [out, in] shape, cut into
 * blocks of ATD_QBLOCK consecutive weights of a row; weight = fp16 scale of
 * its block * its signed code.
 *   ATD_WFMT_DENSE  the matrices in dtype.
 *   ATD_WFMT_Q8     codes int8 [out, in]; scales fp16 [out, in / 32].
 *   ATD_WFMT_Q4     codes 4-bit [out, in / 2] bytes, the code of weight 2i in
 *                   the low nibble of byte i and of weight 2i+1 in the high
 *                   nibble, each stored as code + 8 (codes in [-7, 7]);
 *                   scales fp16 [out, in / 32].
 * Quantized formats need h, Hq*D and F to be multiples of 32 and run every
 * call on the matrix-vector kernels (the dequantization is fused there).
 * quantize_blocks writes both forms from dense weights. */
#define ATD_WFMT_DENSE 0
#define ATD_WFMT_Q8 1
#define ATD_WFMT_Q4 2
#define ATD_QBLOCK 32

/* atd_config.flags: ATD_FLAG_DRY_RUN makes a host-only decoder: every
 * argument check runs and the host state (slot positions, capacities,
 * attached buffers) advances as usual, but no HIP call is made and no
 * device memory is touched.  For validating a decode schedule without a
 * GPU. */
#define ATD_FLAG_DRY_RUN 1
/* ATD_FLAG_NO_MFMA keeps every call on the matrix-vector kernels.  Without it,
 * a decoder with bf16 weights whose h, Hq*D and F are multiples of 32 runs
 * calls of 5 or more rows (batched steps, prefill) in chunks of up to 64 rows
 * through matrix-core GEMMs: activations split into bf16 hi + lo parts, float32
 * accumulation, results within the same tolerance as the vector path. */
#define ATD_FLAG_NO_MFMA 2
/* ATD_FLAG_NO_L2_PREFETCH turns off the weight prefetch of the decode step's
 * attention launch.  Without it, a step that runs on the matrix-vector
 * kernels (fewer than 5 rows, or any step of a decoder without the
 * matrix-core path) and whose attention can span several blocks per row
 * (contexts above 64) appends workgroups to each layer's attention launch that
 * load the O projection's weights, then gate/up blocks, then (where gate/up
 * fit whole) down blocks into the L2 of the XCD whose workgroups will read
 * them next: 24 MiB, or proportionally less where the launch has fewer than
 * 256 (block, KV head) pairs, and nothing where that share cannot take the
 * whole O projection.  Results are identical either way. */
#define ATD_FLAG_NO_L2_PREFETCH 4

/* Device pointers of one layer.  Matrices are row-major [out, in] in the
 * config dtype, or their codes in a quantized weight_format (16-byte
 * aligned); gains and biases are float32. */
typedef struct atd_layer_weights {
  const void* attn_norm; /* [h]            input RMSNorm gain               */
  const void* wq;        /* [Hq*D, h]                                       */
  const void* wk;        /* [Hkv*D, h]                                      */
  const void* wv;        /* [Hkv*D, h]                                      */
  const void* bq;        /* [Hq*D]  or NULL when qkv_bias == 0               */
  const void* bk;        /* [Hkv*D] or NULL                                  */
  const void* bv;        /* [Hkv*D] or NULL                                  */
  const void* q_norm;    /* [D] QK-norm gain of q, or NULL when qk_norm == 0 */
  const void* k_norm;    /* [D] QK-norm gain of k, or NULL                   */
  const void* wo;        /* [h, Hq*D]                                       */
  const void* mlp_norm;  /* [h]            post-attention RMSNorm gain      */
  const void* w_gate;    /* [F, h]                                          */
  const void* w_up;      /* [F, h]                                          */
  const void* w_down;    /* [h, F]                                          */
  /* fp16 block scales [out, in / 32] of the seven matrices when
   * weight_format is quantized (NULL otherwise; 2-byte aligned) */
  const void* wq_scale;
  const void* wk_scale;
  const void* wv_scale;
  const void* wo_scale;
  const void* w_gate_scale;
  const void* w_up_scale;
  const void* w_down_scale;
} atd_layer_weights;

/* All weights of a stack.  The arrays are host arrays of device pointers;
 * they are copied during decoder_create. */
typedef struct atd_weights {
  const atd_layer_weights* layers; /* host [n_layers]                        */
  const void* final_norm;          /* device [h] float32                     */
  const void* const* lm_heads;     /* host [n_lm_heads] -> device [V, h]     */
  const void* const* tables;       /* host [n_tables] -> device [V_g, h]     */
  const int32_t* table_vocab;      /* host [n_tables]: V_g of each table     */
  /* Input projection (qwen3-tts-hip log, Code Predictor stages "prefix
   * projection" / "remaining projection": the Code Predictor of a wider
   * Talker takes its inputs in the Talker's width).  When set, every input
   * row r (input_dim wide: embeddings, extra rows, prefill rows) enters the
   * stack as in_proj r + in_proj_bias.  in_proj: device [hidden, input_dim] in
   * dtype, 16-byte aligned, or NULL (then input_dim must be 0 or hidden);
   * in_proj_bias: device [hidden] float32 or NULL. */
  const void* in_proj;
  const void* in_proj_bias;
} atd_weights;

/* Settings of a sampled token choice (qwen3-tts-hip OPTIMIZATION_LOG: the
 * GenerateOptions defaults top_k 50, top_p 1.0, temperature 0.9, and the
 * device-sampler entry, top_k 1..256).  A draw over one row of logits:
 *   1. the repetition penalty of greedy_argmax on the seen tokens;
 *   2. the top_k largest penalised logits (equal values: lower index first);
 *   3. weights exp((z - z_max) / temperature) over them, in descending order
 *      of logit (equal values: lower index first), summed in that order;
 *   4. the shortest prefix of that order whose weight reaches top_p times the
 *      total (top_p = 1 keeps all top_k);
 *   5. the first candidate whose running weight exceeds u times the prefix's
 *      weight, u in [0, 1) read from `uniforms` (each call states which
 *      entry a draw reads); u so close to 1 that no running weight exceeds
 *      it in float32 takes the prefix's last candidate.
 * top_k = 1 gives greedy_argmax's token.  The random numbers come in from
 * the caller so that a replayed graph and any checker draw the same ones. */
typedef struct atd_sampling {
  int32_t top_k;          /* 1 .. ATD_TOPK_MAX, and <= V */
  float temperature;      /* > 0, finite */
  float top_p;            /* (0, 1] */
  const float* uniforms;  /* device float32 values in [0, 1) */
} atd_sampling;

#define ATD_TOPK_MAX 256

/* Generation controls of the token choices of a sequence ("Qwen3-TTS ncnn
 * port", Talker section: the codes only matched the reference once suppress
 * and min_new_tokens were applied; Audio8-ASR report: decoding runs to EOS).
 * Each choice has an index in its sequence (stated by the call).
 *   suppress        device uint32 bits [B, ceil(V/32)] (bit t of row b = word
 *                   t/32, bit t%32): tokens that are never chosen; or NULL.
 *   eos             the end token, or -1 (then nothing below applies).
 *   min_new_tokens  choices with index < min_new_tokens cannot return eos.
 *   first_index     index of the call's first choice.
 *   eos_step        device int32 [B] or NULL.  -1 while the row runs; the
 *                   choice that returns eos writes its index there, and every
 *                   later choice of the row returns eos without marking the
 *                   seen set.  NULL: eos is chosen like any token, no stop.
 * Suppressed tokens (and a blocked eos) count as logit -inf before the
 * penalty; at least one token of a row must stay choosable.  Decode steps
 * after a stop still run (fed eos): the caller trims at eos_step. */
typedef struct atd_controls {
  const uint32_t* suppress;
  int32_t eos;
  int32_t min_new_tokens;
  int32_t first_index;
  int32_t* eos_step;
} atd_controls;

typedef struct atd_decoder atd_decoder;

/* Create a decoder ("NEON library" page, "Contracts": every argument is
 * validated before any work and a refused call leaves nothing behind;
 * "Rockchip NPU sidecars" page: an unsupported setting is an error, never a
 * silent fallback).  Validates cfg and w (all device pointers non-NULL where
 * required, 16-byte aligned), then allocates its device scratch (residual
 * stream, projections, attention partials, RoPE table, slot tables) sized by
 * max_rows, max_slots and max_ctx: atd_workspace_bytes bytes.  Slots start
 * with no KV buffers attached (attach them with kv_bucket_grow).  *out is set
 * only on ATD_OK.  Errors: INVALID_ARG, SHAPE, DTYPE, UNSUPPORTED, DEVICE. */
int decoder_create(const atd_config* cfg, const atd_weights* w, atd_decoder** out);

/* Device bytes decoder_create allocates for cfg (input_projection: 1 when the
 * weights will carry an input projection).  The decoder owns this scratch
 * rather than taking a caller workspace per call: the graphs that
 * decoder_generate and talker_generate_frames capture hold its addresses, so
 * it has to live exactly as long as the handle.  The query lets a caller
 * budget device memory before creating.  0 for a dry-run config.  Errors:
 * INVALID_ARG and the config errors of decoder_create. */
int atd_workspace_bytes(const atd_config* cfg, int32_t input_projection, size_t* out);

/* Release the decoder and its scratch ("NEON library" page, "Contracts": the
 * caller's storage is never the library's; the weights and KV buffers are
 * untouched).  Waits for work still queued that uses the scratch.  NULL is
 * accepted. */
int decoder_destroy(atd_decoder* dec);

/* Message of the last error on this decoder, or of the last failed
 * decoder_create / greedy_argmax / sample_topk call in this thread when dec
 * is NULL.
 * Valid until the next failing call. */
const char* decoder_last_error(const atd_decoder* dec);

/* Attach KV buffers of capacity s_new rows to `slot` (Audio8-ASR report,
 * dynamic window mechanism).  k_new / v_new: host arrays [n_layers] of
 * device pointers, each [Hkv, s_new, D] in the config kv_dtype, 16-byte
 * aligned.  When the slot already holds buffers, the valid rows
 * [:, :pos, :] of every layer are copied into the new ones on `stream`; the
 * position is kept, so decoding continues at the same token and RoPE
 * position.  The old buffers are the caller's to free once the stream has
 * passed this call.  With no buffers attached yet this is the first attach
 * (position 0).  Errors: INVALID_ARG, CAPACITY (s_new <= pos or
 * s_new > max_ctx), DEVICE. */
int kv_bucket_grow(atd_decoder* dec, int32_t slot, void* const* k_new,
                   void* const* v_new, int32_t s_new, void* stream);

/* Set the number of valid cached rows of `slot` (0 <= pos <= capacity), for
 * caches filled by the caller or resumed from saved buffers.  Enqueued on
 * `stream`.  Errors: INVALID_ARG, CAPACITY, DEVICE. */
int decoder_set_position(atd_decoder* dec, int32_t slot, int32_t pos, void* stream);

/* Host copy of the position and capacity of `slot` (no device access). */
int decoder_get_position(const atd_decoder* dec, int32_t slot, int32_t* pos,
                         int32_t* capacity);

/* Prefill ("qwen3-tts-hip OPTIMIZATION_LOG", Talker and Code Predictor
 * prefill stages; "Audio8-ASR dynamic KV-cache bucket", dynamic window
 * mechanism: the prompt fills cache rows 0..T-1 of the slot's bucket): reset
 * `slot` to position 0 and run the T rows of x (device
 * [T, input_dim] float32; input rows, projected first when the stack has an
 * input projection) at positions 0..T-1 through the stack, each row attending
 * to the rows before it and itself.  Writes KV rows 0..T-1 and leaves the
 * position at T.  Outputs of the last row: y_out (device [h] float32, the
 * final-norm hidden state; may be NULL) and logits_out (device [V]
 * float32) of LM head `head`.  Errors: INVALID_ARG, KV_FULL (T > capacity),
 * CAPACITY (T > max_rows or T > max_ctx), DEVICE. */
int decoder_prefill(atd_decoder* dec, int32_t slot, const float* x, int32_t T,
                    int32_t head, float* y_out, float* logits_out, void* stream);

/* One decode step ("qwen3-tts-hip OPTIMIZATION_LOG", DecodeStepStack entry:
 * per layer the input norm, q/k/v projection, q/k layout and cache write,
 * attention, output projection + residual, post norm, gate/up, SwiGLU, down
 * + residual; "Audio8-ASR dynamic KV-cache bucket", dynamic window mechanism:
 * the step writes row p of the slot's bucket and attends to rows 0..p) of B
 * streams, slots slot0 .. slot0+B-1, each at its own position p.  Input row
 * b = sum over g < G of
 * tables[table_ids[g]][tok[b*G + g]] + extra[b] (extra: device [B, input_dim]
 * float32 or NULL; G may be 0 when extra is given).  tok: device int32
 * [B, G]; ids outside [0, V_g) are clamped into range.  table_ids: host
 * [G].  (With an input projection the row is projected first.)  Writes
 * each slot's KV row p, advances its position by one, and
 * writes y_out (device [B, h] or NULL) and logits_out (device [B, V]) of
 * LM head `head`.  Positions are mirrored on the host, so a full cache is
 * refused before any work: ATD_ERR_KV_FULL, and the caller grows the bucket
 * and retries.  Errors: INVALID_ARG, KV_FULL, CAPACITY, DEVICE. */
int decoder_step(atd_decoder* dec, int32_t slot0, int32_t B, const int32_t* tok,
                 int32_t G, const int32_t* table_ids, const float* extra,
                 int32_t head, float* y_out, float* logits_out, void* stream);

/* decoder_step over any set of slots: row b of tok / extra / y_out /
 * logits_out belongs to slot slots[b] (host int32 [B], distinct, any order),
 * so a batch can step whichever streams are ready ("Audio8-ASR dynamic
 * KV-cache bucket", dynamic window mechanism: the host owns each stream's
 * cache and schedules its steps).  The list is host memory because every slot
 * is validated and its position mirrored on the host before anything is
 * enqueued ("NEON library" page, "Contracts"); the library writes it into its
 * own device scratch on `stream` (kernel arguments, no staging buffer), so the
 * array may be reused once the call returns.  Results equal decoder_step on
 * the same rows.  Errors: as decoder_step, and INVALID_ARG for a NULL list, a
 * slot outside [0, max_slots) or a slot listed twice. */
int decoder_step_slots(atd_decoder* dec, int32_t B, const int32_t* slots, const int32_t* tok,
                       int32_t G, const int32_t* table_ids, const float* extra, int32_t head,
                       float* y_out, float* logits_out, void* stream);

/* Rotary positions apart from the cache position (interleaved multimodal
 * RoPE; "Qwen3-TTS ncnn port", Talker section: the Talker's mRoPE cuts the
 * D/2 rotary frequencies into t / h / w sections [24, 20, 20], interleaved:
 * frequency i follows position i mod 3 while i < 60 and t above).
 * decoder_prefill_mrope is decoder_prefill and decoder_step_mrope is
 * decoder_step, except that row r (a prefill row, or the row of slot
 * slot0 + r) turns its q and k by the positions rope_pos[r] = (t, h, w)
 * (device int32 [T or B, 3]) instead of its cache position: frequency i
 * takes h when i % 3 == 1 and i < 3 s_h, w when i % 3 == 2 and i < 3 s_w,
 * t otherwise, with (s_t, s_h, s_w) = atd_config.mrope_sections
 * (s_t + s_h + s_w = D/2, 3 max(s_h, s_w) <= D/2; {0, 0, 0}: all t).
 * Cache rows, their positions and the attended length are unchanged.  With
 * t = h = w = the cache position the result equals the plain entry point's
 * bit for bit.  Rotary positions are read on the device and clamped into
 * [0, max_ctx) (the angle table's rows).  Errors: as the plain entry
 * points, and INVALID_ARG when rope_pos is NULL. */
int decoder_prefill_mrope(atd_decoder* dec, int32_t slot, const float* x, int32_t T,
                          const int32_t* rope_pos, int32_t head, float* y_out,
                          float* logits_out, void* stream);
int decoder_step_mrope(atd_decoder* dec, int32_t slot0, int32_t B, const int32_t* tok,
                       int32_t G, const int32_t* table_ids, const float* extra,
                       const int32_t* rope_pos, int32_t head, float* y_out,
                       float* logits_out, void* stream);

/* The input-embedding part of decoder_step alone: x_out (device [B, input_dim]
 * float32) = sum_g tables[table_ids[g]][tok[b*G+g]] + extra[b].  Used to
 * build prefill rows from device-resident tokens.  Errors: INVALID_ARG,
 * CAPACITY, DEVICE. */
int decoder_embed(atd_decoder* dec, int32_t B, const int32_t* tok, int32_t G,
                  const int32_t* table_ids, const float* extra, float* x_out,
                  void* stream);

/* Greedy token with repetition penalty (qwen3-tts-hip log, penalty entry;
 * ncnn port, Talker section).  For each row b of logits (device [B, V]
 * float32): logits of tokens whose bit is set in seen (device uint32
 * [B, ceil(V/32)], bit t of row b = word t/32, bit t%32; may be NULL) are
 * divided by `penalty` when positive and multiplied by it otherwise; the
 * token is the lowest index of the maximum; margin = best - second best
 * (0 on a tie).  Writes tok_out (device int32 [B]) and margin_out (device
 * float32 [B] or NULL) and sets the chosen token's bit in seen.  The logits
 * are not modified.  controls (or NULL): atd_controls, the choice of every
 * row having index controls->first_index.  Uses a device scratch buffer
 * that the library keeps per device (allocated on first use; a call that
 * needs more space gets a larger one, and earlier ones stay allocated until
 * the process ends, so a graph captured around an earlier call stays valid).
 * Two calls that overlap on different streams of one device share it and
 * race.  Errors: INVALID_ARG, DEVICE. */
int greedy_argmax(const float* logits, int32_t B, int32_t V, uint32_t* seen,
                  float penalty, const atd_controls* controls, int32_t* tok_out,
                  float* margin_out, void* stream);

/* greedy_argmax for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and results as greedy_argmax (bit for bit), but its per-row
 * partials live in a fixed device array of the library (256 KB on each GPU
 * it runs on, held until the process ends) instead of a buffer allocated on
 * first use: the call allocates nothing.  B * ceil(V / 4096) * 3 may not
 * exceed 65536 (e.g. 574 rows of a 151936-token vocabulary), else
 * ATD_ERR_CAPACITY.  Every call on one GPU shares that array and it keeps
 * the last call's partials: calls that overlap on one GPU (on different
 * streams) race.  Errors: as greedy_argmax, and CAPACITY. */
int greedy_argmax_noalloc(const float* logits, int32_t B, int32_t V, uint32_t* seen,
                          float penalty, const atd_controls* controls, int32_t* tok_out,
                          float* margin_out, void* stream);

/* Sampled token per row (the draw of atd_sampling; qwen3-tts-hip log,
 * device-sampler entry).  logits device [B, V] float32; seen and penalty as
 * in greedy_argmax (the chosen token's bit is set); row b draws
 * sampling->uniforms[b] (device [B]).  Writes tok_out (device int32 [B]).
 * Rows of up to 8192 logits run in one workgroup each; longer rows first
 * reduce each 8192-logit chunk to its top_k candidates, which needs
 * ceil(V / 8192) * top_k <= 8192.  controls as in greedy_argmax.  Uses the
 * per-device scratch buffer of greedy_argmax.  Errors: INVALID_ARG, UNSUPPORTED (V too long for top_k),
 * DEVICE. */
int sample_topk(const float* logits, int32_t B, int32_t V, uint32_t* seen, float penalty,
                const atd_sampling* sampling, const atd_controls* controls,
                int32_t* tok_out, void* stream);


/* Generation on the device: n_steps decode steps of `slot` with the token
 * fed back without a host round trip (the qwen3-tts-hip log measures the
 * host-side sampling and token copies as the remaining host cost).  Step k
 * embeds tok_io[0..G-1] from tables table_ids (host [G]) plus extra
 * (device [h] or NULL, the same every step), runs the stack and LM head
 * `head`, then chooses the token over `seen` (device [ceil(V/32)] or NULL)
 * and `penalty`: the penalized argmax of greedy_argmax when sampling is
 * NULL, else the draw of atd_sampling with u = sampling->uniforms[k]
 * (device [n_steps]); controls (or NULL) as in atd_controls, step k being
 * choice controls->first_index + k.  The token goes to tok_io[0] (the other
 * G-1 ids are held) and, when tokens_out is not NULL, to tokens_out[k]
 * (device int32 [n_steps]).  y_out (device [h] or NULL) and logits_out
 * (device [V]) hold the last step's outputs.  The launches of one step are
 * captured once into a HIP graph and replayed; the graph is cached for this
 * argument set (sampling settings and uniforms pointer included) and
 * bucket and rebuilt when either changes.  Refused with ATD_ERR_KV_FULL when
 * pos + n_steps exceeds the slot's capacity (grow the bucket first; nothing
 * runs).  Errors: INVALID_ARG, KV_FULL, CAPACITY, UNSUPPORTED (a sampled
 * vocabulary too long for top_k, see sample_topk), DEVICE. */
int decoder_generate(atd_decoder* dec, int32_t slot, int32_t n_steps, int32_t* tok_io,
                     int32_t G, const int32_t* table_ids, const float* extra, int32_t head,
                     uint32_t* seen, float penalty, const atd_sampling* sampling,
                     const atd_controls* controls, int32_t* tokens_out, float* y_out,
                     float* logits_out, void* stream);

/* The Talker's two-level frame loop on the device ("Qwen3-TTS ncnn port",
 * section "Talker: non-standard structure and two-level generation"; the
 * qwen3-tts-hip OPTIMIZATION_LOG's Code Predictor stages).  Runs n_frames
 * frames, captured as HIP graphs on first use and replayed.  Frame f:
 *   - unless f = 0, one Talker step (decoder tk, slot tk_slot) fed
 *     sum_{g<16} table_g[c_g] + text[f] (the previous frame's codes), head 0:
 *     writes y_io and tk_logits; the choice over `seen` with `penalty`
 *     gives the frame's c0: greedy (greedy_argmax rules) when tk_sampling
 *     is NULL, else the draw of atd_sampling with
 *     u = tk_sampling->uniforms[f];
 *   - the Code Predictor pass (decoder cp, slot cp_slot, restarted at
 *     position 0): a 2-row prefill of [y_io, table_0[c0]] with head 0 gives
 *     c1, then steps j = 1..14 fed table_j[c_j] with head j give c_{j+1};
 *     no penalty; greedy when cp_sampling is NULL, else the draw with
 *     u = cp_sampling->uniforms[f * 15 + j] for c_{j+1} (the log's
 *     "subtalker" settings);
 *   - the frame's 16 codes are appended to codes_out.
 * codes_io   [16] int32 device.  On entry codes_io[0] is frame 0's c0 (the code
 *            the caller chose from its prefill, already marked in `seen`).
 *            On return it holds the last frame's codes.
 * y_io       [h] float32 device, 16-byte aligned.  On entry the Talker
 *            final-norm output that goes with frame 0's c0.  On return the last
 *            Talker step's output.
 * text       [n_frames, h] float32 device; row f is added to frame f's Talker
 *            input (row 0 unused; may be NULL when n_frames = 1).
 * seen       [ceil(V_tk / 32)] uint32 device, updated; penalty > 0.
 * tk_sampling uniforms: device [n_frames] (entry 0 unused); cp_sampling
 *            uniforms: device [n_frames, 15].  Both settings belong to the
 *            captured graphs' key.
 * tk_controls the Talker's atd_controls (or NULL): frame f's c0 (f >= 1) is
 *            choice first_index + f; after a stop c0 stays eos (the frames
 *            still run: trim at eos_step).
 * codes_out  [n_frames, 16] int32 device, or NULL.
 * tk_logits  [V_tk] and cp_logits [V_cp] float32 device: the last logits of
 *            each decoder.
 * Requirements: equal hidden sizes; tk has >= 16 tables (table g: codes of
 * group g); cp has >= 15 tables and >= 15 LM heads (table 0 must be the
 * Talker's code table); cp_slot holds >= 16 rows and cp max_rows >= 2;
 * tk_slot has room for n_frames - 1 more rows (no bucket growth inside).
 * Afterwards tk_slot has advanced n_frames - 1 rows and cp_slot is at 16.
 * Each of the two decoders' scratch is used, so neither may run other work
 * concurrently.  Errors: INVALID_ARG, SHAPE, CAPACITY, KV_FULL, UNSUPPORTED,
 * DEVICE. */
int talker_generate_frames(atd_decoder* tk, int32_t tk_slot, atd_decoder* cp, int32_t cp_slot,
                           int32_t n_frames, int32_t* codes_io, float* y_io, const float* text,
                           uint32_t* seen, float penalty, const atd_sampling* tk_sampling,
                           const atd_sampling* cp_sampling, const atd_controls* tk_controls,
                           int32_t* codes_out, float* tk_logits, float* cp_logits, void* stream);

/* Block quantization of dense weights into a quantized weight_format
 * (ATD_WFMT_Q8 or ATD_WFMT_Q4; the formats are described with
 * atd_config.weight_format).  w: device [rows, cols] in dtype (ATD_F32 or
 * ATD_BF16), 16-byte aligned, cols a multiple of 32.  For each block of 32
 * weights of a row: d = max|w| / 127 (Q8) or / 7 (Q4) in float32; code =
 * w / d (float32 division) rounded to the nearest integer, halves away from
 * zero, clamped to +-127 (+-7), 0 when d = 0; the scale stored is d rounded
 * to fp16 (nearest even).  Writes codes (device, 16-byte aligned: rows * cols
 * bytes for Q8, rows * cols / 2 for Q4) and scales (device uint16 [rows,
 * cols / 32]) on `stream`.  Errors: INVALID_ARG, DTYPE, SHAPE, DEVICE. */
int quantize_blocks(const void* w, int32_t dtype, int64_t rows, int32_t cols, int32_t format,
                    void* codes, uint16_t* scales, void* stream);

/* Codec decoder convolutions (qwen3-tts-hip OPTIMIZATION_LOG, codec entries:
 * the decoder's time goes to a dilated causal convolution and a transposed
 * convolution, the latter rewritten by output phase as GEMMs over prepacked
 * weights).  float32, channel-major [channels, frames], device pointers
 * 4-byte aligned; the outputs may not overlap the inputs.
 *
 * codec_conv1d_causal: y[co, t] = bias[co] + sum over ci < cin, j < K of
 *   w[co, ci, j] * x[ci, t - (K-1-j) * dilation], x = 0 before frame 0.
 *   x [cin, T], w [cout, cin, K], bias [cout] or NULL, y [cout, T]; with
 *   accumulate = 1 the result is added to y (a residual connection).
 * codec_transconv1d_pack: the weights of a transposed convolution with
 *   kernel 2 * stride, w [cin, cout, 2 * stride], rearranged once (at load
 *   time) into packed [stride, cout, cin * 2] for codec_transconv1d.
 * codec_transconv1d: y[co, t * stride + p] = bias[co] + sum over ci of
 *   w[ci, co, p] x[ci, t] + w[ci, co, p + stride] x[ci, t - 1] (x[., -1] = 0)
 *   for t < T, p < stride: the transposed convolution's first T * stride
 *   outputs.  x [cin, T], y [cout, T * stride].
 * Errors: INVALID_ARG (NULL / misaligned pointer, sizes < 1, cin * K or a
 * tensor beyond 2^31 elements), DEVICE. */
int codec_conv1d_causal(const float* x, const float* w, const float* bias, int32_t cin,
                        int32_t cout, int32_t T, int32_t K, int32_t dilation, int32_t accumulate,
                        float* y, void* stream);
int codec_transconv1d_pack(const float* w, int32_t cin, int32_t cout, int32_t stride,
                           float* packed, void* stream);
int codec_transconv1d(const float* x, const float* packed, const float* bias, int32_t cin,
                      int32_t cout, int32_t T, int32_t stride, float* y, void* stream);

/* Stages of a decode step, for decoder_time_stage. */
enum {
  ATD_STAGE_QKV = 0,     /* RMSNorm + q/k/v projection                       */
  ATD_STAGE_ROPE = 1,    /* QK norm + RoPE + cache append of a prefill block  */
  ATD_STAGE_ATTN = 2,    /* split-K attention, its splits merged in the same
                            launch (for decode steps it also applies the QK
                            norm + RoPE and appends the new cache row)       */
  ATD_STAGE_OPROJ = 3,   /* output projection + residual                      */
  ATD_STAGE_GATEUP = 4,  /* RMSNorm + gate/up projection + SwiGLU             */
  ATD_STAGE_DOWN = 5,    /* down projection + residual                        */
  ATD_STAGE_HEAD = 6,    /* final RMSNorm + LM head                           */
  ATD_STAGE_COUNT = 7
};

/* Measurement: enqueue the kernels of one per-layer stage (ATD_STAGE_QKV,
 * _ATTN, _OPROJ, _GATEUP or _DOWN) of a decode step of the B rows on slots
 * slot0 .. slot0+B-1 (the launch shapes of decoder_step with those rows:
 * the vector kernels for B <= 2, the 64-row matrix-core chunks otherwise)
 * for every layer in turn (each layer's weights once, as in a step), `reps`
 * times, between two HIP events recorded on `stream`, and return the mean
 * time of the stage per layer in microseconds.  The kernels read and write
 * the decoder's own scratch (the residual stream they update there is
 * rebuilt by the next step or prefill); ATD_STAGE_ATTN also writes the
 * not-yet-valid cache row at each slot's write position, which the next
 * step overwrites (so it needs each slot's position below its capacity).
 * Slot positions do not move.  Waits for the stream.
 * Errors: INVALID_ARG, CAPACITY, KV_FULL, DEVICE. */
int decoder_time_stage(atd_decoder* dec, int32_t stage, int32_t slot0, int32_t B,
                       int32_t reps, void* stream, double* us_per_layer);

/* Measurement: the attainable read bandwidth of this device ("Rockchip NPU
 * sidecars" page: a DRAM-bound decode is judged against a measured read
 * ceiling, taken over a working set larger than the caches).  Reads the
 * `bytes` at buf (device, 16-byte aligned, a multiple of 16; pass more than
 * the 256 MB memory-side cache) once as a warm-up and then `reps` times with
 * a grid-stride streaming kernel of 16-byte loads, between two HIP events on
 * `stream`, and returns the mean microseconds of one read (bytes / that time
 * is the attainable bandwidth).  sink: device uint32 scratch the kernel may
 * write (its value means nothing).  Waits for the stream.  Errors:
 * INVALID_ARG, DEVICE. */
int atd_read_stream(const void* buf, size_t bytes, int32_t reps, uint32_t* sink, void* stream,
                    double* us_per_read);

#ifdef __cplusplus
}
#endif

#endif /* ATD_H */
