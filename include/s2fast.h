/*
 * s2fast — the Fast-AR codebook decoder of the Dual-AR (Fish Audio S2 Pro)
 * text-to-speech model, as one HIP library for AMD Instinct MI355X (gfx950).
 *
 * What it computes ("Fast-AR codebook decoding and the generation main loop",
 * s2.cpp analysis pages, sections 1-5; Mizuoto "Fish Speech" engine page,
 * section "What matches upstream"):
 *   For every frame, codebook 0 is the semantic code (the Slow-AR main token
 *   minus semantic_begin, clamped into the codebook).  Then, for k = 1..9, a
 *   4-layer causal GQA transformer runs over the window
 *       [hidden, fast_embeddings[c_0], ..., fast_embeddings[c_{k-1}]]
 *   (positions restart at 0 on every call, causal mask offset 0, no KV cache
 *   in the method's definition), its last position goes through fast_norm
 *   and the untied fast_output matrix to give codebook_size logits, and a
 *   sampler turns the logits into c_k.  Output: 10 codes per frame.
 *
 * Conventions used by every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *     tensors) unless stated otherwise.  The caller owns them.
 *   - Matrices are row-major [out, in]; vectors are contiguous.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Entry points only enqueue work on it; nothing blocks the host except
 *     where stated.  The caller synchronises before reading outputs.
 *   - Return value: S2FAST_OK (0) or a positive S2FAST_ERR_* code.  Argument
 *     errors are detected on the host before anything is enqueued, and then
 *     no output is touched.
 *   - One context may be used by one host thread and one stream at a time;
 *     calls that overlap on one context race.
 */
#ifndef S2FAST_H
#define S2FAST_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  S2FAST_OK = 0,
  S2FAST_ERR_ARG = 1,              /* NULL pointer, bad size or unsupported shape */
  S2FAST_ERR_NO_FAST_DECODER = 2,  /* a required Fast-AR weight pointer is NULL
                                      (the pages' "model has no fast decoder") */
  S2FAST_ERR_HIDDEN_DIM = 3,       /* hidden width differs from the model's in_dim */
  S2FAST_ERR_PREFIX_LEN = 4,       /* prefix would be >= num_codebooks codes */
  S2FAST_ERR_BATCH = 5,            /* B < 1 or B > max_batch */
  S2FAST_ERR_HIP = 6,              /* a HIP runtime call failed */
  S2FAST_ERR_NOMEM = 7,            /* device or host allocation failed */
  S2FAST_ERR_DEVICE = 8,           /* device not supported (not gfx950, or the
                                      grid cannot be co-resident) */
  S2FAST_ERR_SCRATCH = 9           /* the shape needs more scratch than the
                                      static buffer of s2fast_decode_frame_static */
};

/* Weight types.  S2FAST_Q8: weight-only int8 — every weight matrix (wqkv,
 * wo, w1, w3, w2, fast_output, fast_project_in) is int8 [out, in] with one
 * float32 scale per output row, W[r, k] = scale[r] * q[r, k] (the pages name
 * GGUF quantised tensors, "Overall architecture & Dual-AR data flow",
 * section 5 and "Model loading and GGUF", section 4, but no Fast-AR
 * format; per-row symmetric int8 is this library's choice); norm weights
 * and fast_embeddings are bf16.  Q8 contexts decode every request with the
 * batch-1 kernel (one launch per request). */
enum { S2FAST_BF16 = 0, S2FAST_F32 = 1, S2FAST_Q8 = 2 };

/* Model shape ("Overall architecture & Dual-AR data flow", section 2;
 * "Model loading and GGUF", section 2.2).  S2 Pro: in_dim 2560, dim 2560,
 * 4 layers, 32 query / 8 KV heads, head_dim 128, ffn 9728, codebook 4096,
 * 10 codebooks, context 11, RoPE base 1e6, eps 1e-6. */
typedef struct s2fast_config {
  int32_t in_dim;          /* width of the Slow-AR hidden state */
  int32_t dim;             /* fast_dim */
  int32_t n_layer;         /* <= S2FAST_MAX_LAYERS */
  int32_t n_head;          /* query heads */
  int32_t n_head_kv;       /* key/value heads; n_head % n_head_kv == 0 */
  int32_t head_dim;        /* multiple of 8, <= 128 */
  int32_t ffn_dim;         /* SwiGLU hidden width */
  int32_t codebook_size;   /* V: logits per call, <= 8192 */
  int32_t num_codebooks;   /* codes per frame (10): num_codebooks-1 decode steps */
  int32_t context;         /* RoPE positions (11); must be >= num_codebooks */
  float rope_base;         /* 1e6 */
  float norm_eps;          /* 1e-6, also used by the per-head q/k norms */
  int32_t has_project_in;  /* fast_project_in [dim, in_dim] present */
  int32_t has_qk_norm;     /* per-head q_norm / k_norm present */
  int32_t weight_dtype;    /* S2FAST_BF16 or S2FAST_F32 (all matrices and norm
                              weights share it), or S2FAST_Q8 (int8 matrices,
                              bf16 vectors; widths multiples of 16) */
  int32_t max_batch;       /* largest B passed to the decode calls */
} s2fast_config;

#define S2FAST_MAX_LAYERS 8

/* Tensor names follow the GGUF Fast-AR set ("Model loading and GGUF",
 * section 3).  All pointers are device pointers of `weight_dtype`, row-major
 * [out, in].  They must stay valid and unchanged for the context's life;
 * the library reads them in place.  At creation it also derives one table
 * from them: the layer-0 q/k/v of every embedding row,
 * wqkv . (attention_norm * e_c) / rms(e_c) for c < codebook_size, float32
 * [codebook_size, qkv width] (100 MB at the S2 Pro shape).  A decode step
 * after the first adds one embedding row, so its layer-0 projection is a
 * row of this table instead of a pass over wqkv. */
typedef struct s2fast_layer_weights {
  const void* attention_norm;  /* [dim] */
  const void* wqkv;            /* [(n_head + 2 n_head_kv) head_dim, dim]; rows are
                                  Q heads, then K heads, then V heads */
  const void* q_norm;          /* [head_dim], NULL iff !has_qk_norm */
  const void* k_norm;          /* [head_dim], NULL iff !has_qk_norm */
  const void* wo;              /* [dim, n_head head_dim] */
  const void* ffn_norm;        /* [dim] */
  const void* w1;              /* [ffn_dim, dim] gate */
  const void* w3;              /* [ffn_dim, dim] up */
  const void* w2;              /* [dim, ffn_dim] down */
} s2fast_layer_weights;

/* Row scales of an S2FAST_Q8 model's matrices: float32 device vectors, one
 * value per output row of the matrix named. */
typedef struct s2fast_q8_layer_scales {
  const float* wqkv;           /* [(n_head + 2 n_head_kv) head_dim] */
  const float* wo;             /* [dim] */
  const float* w1;             /* [ffn_dim] */
  const float* w3;             /* [ffn_dim] */
  const float* w2;             /* [dim] */
} s2fast_q8_layer_scales;

typedef struct s2fast_q8_scales {
  const float* project_in;     /* [dim], NULL iff !has_project_in */
  const float* output;         /* [codebook_size] */
  s2fast_q8_layer_scales layers[S2FAST_MAX_LAYERS];
} s2fast_q8_scales;

typedef struct s2fast_weights {
  const void* project_in;      /* fast_project_in [dim, in_dim], NULL iff !has_project_in */
  const void* embeddings;      /* fast_embeddings [codebook_size, dim] */
  const void* norm;            /* fast_norm [dim] */
  const void* output;          /* fast_output [codebook_size, dim] (untied) */
  s2fast_layer_weights layers[S2FAST_MAX_LAYERS];
  const s2fast_q8_scales* q8_scales;   /* HOST pointer to the row scales of an
                                          S2FAST_Q8 model (copied at creation),
                                          NULL for the other weight types */
} s2fast_weights;

typedef struct s2fast_ctx s2fast_ctx;

/* Create a decoder over the caller's Fast-AR weights: the device side of
 * the pages' model load for the fast decoder ("Model loading and GGUF",
 * sections 3 and 4: the fast_* tensors are bound by name and kept on the
 * GPU, where the Fast-AR runs every frame).
 * Validate the shape and the weight pointers, allocate the context's device
 * scratch for max_batch requests, build the bf16-rounded RoPE table and the
 * layer-0 q/k/v table above (one GEMM on the current stream's device,
 * synchronised before returning).  With max_batch >= 2 the context also
 * keeps a repacked copy of every weight matrix for the batched kernel (the
 * size of the weights: 0.83 GB at the S2 Pro shape), in which each
 * workgroup's rows form one contiguous stream; batches run 64 requests to a
 * launch.
 * Uses the current HIP device.  On success *out owns the scratch; release
 * it with s2fast_destroy.  Shape limits (else S2FAST_ERR_ARG): dim, in_dim,
 * ffn_dim and the per-KV-group width (n_head/n_head_kv)*head_dim are
 * multiples of 8 (bf16) or 4 (f32) elements; dim, in_dim, ffn_dim <= 16384;
 * head_dim a multiple of 8 and <= 128; context <= 16; 2 <= num_codebooks <= context;
 * codebook_size <= 8192; n_head_kv <= 64.
 * Missing required weight pointers (or, for S2FAST_Q8, row scales) give
 * S2FAST_ERR_NO_FAST_DECODER; q8_scales with another weight type gives
 * S2FAST_ERR_ARG. */
int s2fast_create(const s2fast_config* cfg, const s2fast_weights* w, s2fast_ctx** out);

/* Wait for the device, then free everything the context owns (not the
 * caller's weights).  NULL is ignored. */
void s2fast_destroy(s2fast_ctx* ctx);

/* Static description of an S2FAST_* code (never NULL). */
const char* s2fast_strerror(int code);

/* Device-side failure report.  Every grid-wide wait inside a launch is
 * bounded; if one gives up, the launch ends early and its last block
 * restores the context's state for the next launch and applies the main
 * loop's convention for a failed Fast-AR call ("Fast-AR codebook decoding
 * ...", section 5.2): every request of that launch keeps codes[:, 0] (its
 * clamped semantic code) and gets codes[:, 1:] = 0; logits of a
 * teacher-forced launch are then undefined.  This call waits for the work
 * enqueued on `stream`, returns S2FAST_ERR_HIP if any launch on this context
 * failed that way since the previous call (and clears the report), else
 * S2FAST_OK.  Blocking. */
int s2fast_status(s2fast_ctx* ctx, void* stream);

/* Decode one frame for B requests ("Fast-AR codebook decoding ...", section
 * 5.1, step 3).
 *   hidden      [B, in_dim]  f32  Slow-AR hidden state (already normalised);
 *                                 16-byte aligned device memory
 *   sem_code    [B]          i32  main_token - semantic_begin; clamped on the
 *                                 device to [0, codebook_size-1] (section 5.2)
 *   uniforms    [B, num_codebooks-1] f32  one uniform in (0,1) per draw;
 *                                 column k-1 drives codebook k.  Each draw
 *                                 expands it into one exponential per top-k
 *                                 candidate with SplitMix64 (see the sampler
 *                                 below)
 *   temperature [B] f32  <= 0 (or NaN) decodes greedily
 *   top_p       [B] f32  nucleus mass; the smallest prefix of the sorted
 *                        top-k set with cumulative probability >= top_p
 *   top_k       [B] i32  clamped on the device to [1, min(V, 64)]
 *   codes       [B, num_codebooks] i32 OUT  [sem_code, c_1, ..., c_9]
 * Sampler (Mizuoto page, "What matches upstream": argmax(probs / -log u), top-k 30):
 *   candidates = the top_k largest logits (value desc, index asc);
 *   z = l / T; e_j = f32(exp(f64(z_j - z_0))); p_j = e_j / sum (f32, rank
 *   order); keep ranks 0..m, m = first j with cumulative p >= top_p;
 *   u_j = (floor(splitmix64(bits(u) * 2^32 + j) / 2^40) + 0.5) * 2^-24;
 *   code = kept candidate maximising p_j / f32(-log(f64(u_j))).
 * Errors: S2FAST_ERR_BATCH for B outside [1, max_batch]; S2FAST_ERR_ARG for
 * NULL pointers or a hidden pointer that is not 16-byte aligned.  Batches
 * run as launches of up to 64 requests (the context's group size); if a
 * launch cannot be enqueued, codes[:, 1:] of its requests and of every
 * later one are zero-filled on `stream` (the main loop's "failed
 * fast_decode fills the rest of the frame with 0" convention, section 5.2)
 * and S2FAST_ERR_HIP is returned; earlier launches keep their codes.  A
 * failure inside a launch is reported by s2fast_status. */
int s2fast_decode_frame(s2fast_ctx* ctx, int32_t B, const float* hidden, const int32_t* sem_code,
                        const float* uniforms, const float* temperature, const float* top_p,
                        const int32_t* top_k, int32_t* codes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * s2fast_decode_frame with the same arguments and results for every request
 * as a batch-1 call of s2fast_decode_frame (each request runs the batch-1
 * kernel, one launch after another), whose per-frame scratch (activations,
 * attention accumulators, the frame's keys and values, logits, barrier
 * flags) lives in one static 16 MiB device array per GPU instead of the
 * context's arena.  It calls no allocating routine: the first call on a
 * device takes the array's device address and clears it with a kernel on
 * `stream` (the array then stays with the process), and so does the first
 * call after one with a context of another shape.  The context must have
 * been created on the current device (else S2FAST_ERR_DEVICE); a shape
 * whose batch-1 arena exceeds 16 MiB gives S2FAST_ERR_SCRATCH (the S2 Pro
 * shape needs 12.2 MiB).  Every call on one GPU shares the array: calls that
 * overlap on one GPU, from any context or thread, race, and must be
 * serialised by the caller (one stream).  Each call leaves the array ready
 * for the next, also after a failure reported by s2fast_status.  Other
 * errors as s2fast_decode_frame. */
int s2fast_decode_frame_static(s2fast_ctx* ctx, int32_t B, const float* hidden, const int32_t* sem_code,
                               const float* uniforms, const float* temperature, const float* top_p,
                               const int32_t* top_k, int32_t* codes, void* stream);

/* Teacher-forced logits of a whole frame (the per-step logits the main
 * loop hands to the sampler, "Fast-AR codebook decoding ...", section 4):
 * for k = 1..num_codebooks-1 the prefix is
 * codes[:, 0..k-1] (codes[:, 0] is clamped like sem_code; the last column
 * is not read) and logits[:, k-1, :] receives the codebook_size logits of
 * that call.
 *   hidden [B, in_dim] f32, 16-byte aligned; codes [B, num_codebooks] i32
 *   (each in [0, V));
 *   logits [B, num_codebooks-1, codebook_size] f32 OUT.
 * Out-of-range prefix codes are clamped to [0, V-1] on the device. */
int s2fast_forward_logits(s2fast_ctx* ctx, int32_t B, const float* hidden, const int32_t* codes,
                          float* logits, void* stream);

/* One Fast-AR call as the pages define it ("Fast-AR codebook decoding ...",
 * sections 1-4): the codebook_size logits that follow `prefix` for each of
 * B requests, the window being [hidden, fast_embeddings[prefix[0]], ...].
 *   hidden     [B, hidden_dim] f32, 16-byte aligned
 *   hidden_dim must equal the model's in_dim, else S2FAST_ERR_HIDDEN_DIM
 *   prefix     [B, prefix_len] i32 codes (prefix[:, 0] is the semantic code;
 *              every code is clamped on the device into [0, codebook_size))
 *   prefix_len 1 <= prefix_len < num_codebooks, else S2FAST_ERR_PREFIX_LEN
 *   logits     [B, codebook_size] f32 OUT
 * Checks run in the pages' order (hidden width, then prefix length), then
 * S2FAST_ERR_BATCH and S2FAST_ERR_ARG; nothing is enqueued on an error. */
int s2fast_fast_decode(s2fast_ctx* ctx, int32_t B, const float* hidden, int32_t hidden_dim, const int32_t* prefix,
                       int32_t prefix_len, float* logits, void* stream);

/* ---- Slow-AR decode step and the full Dual-AR frame ----
 *
 * What a step computes ("Overall architecture & Dual-AR data flow", sections
 * 3.2 and 3.4; "Fast-AR codebook decoding and the generation main loop",
 * sections 5 and 6): the previous frame's 11 values (main token m and codes
 * c_0..c_9) give the input
 *     x = (1/sqrt(num_codebooks+1)) * embeddings[m]
 *         + sum_j codebook_embeddings[j * codebook_size + c_j],
 * (the codebook terms count only when m is a semantic id: the prompt's
 * mask; a generated frame's main token is one), which runs through n_layer
 * pre-norm layers (RMSNorm, fused wqkv, per-head
 * q/k RMSNorm, pair RoPE at position n_past, GQA attention over the KV cache
 * positions 0..n_past, wo, SwiGLU) as position n_past; the layer's new key
 * and value are written into the cache at n_past.  hidden = RMSNorm(x, norm);
 * the tied logits embeddings . hidden are masked to the semantic ids
 * [semantic_begin, semantic_begin + codebook_size) and end_id, and the main
 * token is drawn from them with the sampler of s2fast_decode_frame.  A
 * semantic main token already in the window of the last 10 main tokens is
 * drawn again at temperature 1.0, top_p 0.9 (same top_k) with the second
 * uniform; the window then receives the main token.
 * Only the unmasked logits are computed: every other logit is -inf and can
 * never be drawn. */
#define S2FAST_SLOW_MAX_LAYERS 64
#define S2FAST_RAS_WINDOW 10

/* S2 Pro: dim 2560, 36 layers, 32 / 8 heads, head_dim 128, ffn 9728, vocab
 * 155776, codebook_size 4096, 10 codebooks, semantic ids 151678..155773,
 * RoPE base 1e6, eps 1e-6 ("Model loading and GGUF", section 2.2). */
typedef struct s2fast_slow_config {
  int32_t dim;
  int32_t n_layer;          /* <= S2FAST_SLOW_MAX_LAYERS */
  int32_t n_head;
  int32_t n_head_kv;        /* n_head % n_head_kv == 0, n_head / n_head_kv <= 8 */
  int32_t head_dim;         /* multiple of 8, <= 128 */
  int32_t ffn_dim;
  int32_t vocab;            /* rows of embeddings */
  int32_t codebook_size;    /* semantic ids and codes per codebook, <= 8191 */
  int32_t num_codebooks;    /* codes per frame, 1..10 */
  int32_t semantic_begin;   /* first semantic id */
  int32_t end_id;           /* the end-of-speech id sem_mask also leaves open */
  int32_t max_context;      /* positions the KV cache holds */
  float rope_base;
  float norm_eps;
  int32_t has_qk_norm;
  int32_t weight_dtype;     /* S2FAST_BF16 or S2FAST_F32: weights and KV cache */
} s2fast_slow_config;

/* Device pointers of weight_dtype, row-major [out, in], valid and unchanged
 * for the context's life. */
typedef struct s2fast_slow_weights {
  const void* embeddings;           /* [vocab, dim], also the tied output matrix */
  const void* codebook_embeddings;  /* [num_codebooks * codebook_size, dim] */
  const void* norm;                 /* [dim] final RMSNorm weight */
  s2fast_layer_weights layers[S2FAST_SLOW_MAX_LAYERS];
} s2fast_slow_weights;

typedef struct s2fast_slow_ctx s2fast_slow_ctx;

/* Create a Slow-AR step over the caller's weights ("Model loading and
 * GGUF", section 3: the Slow-AR tensors; "Overall architecture ...", section
 * 2: the 36-layer shape).
 * Validate, allocate the step's device scratch (one launch's arena, about
 * n_layer * 0.7 MB at the S2 Pro shape) and the RoPE table for max_context
 * positions.  Shape limits (else S2FAST_ERR_ARG): dim, ffn_dim and the
 * per-KV-group width multiples of 8 (bf16) or 4 (f32) elements and <= 16384;
 * the semantic range inside [0, vocab); end_id in [0, vocab);
 * max_context >= 1.  Missing weight pointers give S2FAST_ERR_NO_FAST_DECODER.
 * Release with s2fast_slow_destroy. */
int s2fast_slow_create(const s2fast_slow_config* cfg, const s2fast_slow_weights* w, s2fast_slow_ctx** out);

/* Wait for the device, then free the context (not the caller's weights). */
void s2fast_slow_destroy(s2fast_slow_ctx* ctx);

/* As s2fast_status, for Slow-AR launches: a step or prefill launch whose
 * bounded grid-wide wait gave up draws no main token and leaves the window
 * unchanged; hidden_out, the cache entry at its position and logits_out are
 * then undefined.  Blocking. */
int s2fast_slow_status(s2fast_slow_ctx* ctx, void* stream);

/* One Slow-AR decode step of one request.
 *   kv_cache    [n_layer, n_head_kv, max_context, 2, head_dim] weight_dtype,
 *               keys (after q/k norm and RoPE) then values per position,
 *               16-byte aligned; positions < n_past are read, position n_past
 *               is written (new entries are rounded to the cache type)
 *   n_past      host int in [0, max_context): the new position's index
 *   prev_main   [1] i32, prev_codes [num_codebooks] i32: the previous
 *               frame's values (clamped on the device into [0, vocab) and
 *               [0, codebook_size))
 *   window      [1 + S2FAST_RAS_WINDOW] i32 IN/OUT: count, then the last
 *               main tokens oldest first
 *   u           [2] f32 uniforms in (0,1): the draw and the repetition redraw
 *   temperature, top_p [1] f32, top_k [1] i32: as s2fast_decode_frame
 *   main_out    [1] i32 OUT the main token
 *   sem_code_out [1] i32 OUT main - semantic_begin clamped to [0, codebook_size)
 *   hidden_out  [dim] f32 OUT RMSNorm(x, norm), 16-byte aligned
 *   logits_out  [n_allowed] f32 OUT or NULL: the unmasked logits, ids
 *               ascending (n_allowed = codebook_size, + 1 if end_id is
 *               outside the semantic range)
 * Errors: S2FAST_ERR_ARG for NULL pointers (other than logits_out),
 * misaligned kv_cache / hidden_out or n_past outside [0, max_context). */
int s2fast_slow_step(s2fast_slow_ctx* ctx, void* kv_cache, int32_t n_past, const int32_t* prev_main,
                     const int32_t* prev_codes, int32_t* window, const float* u, const float* temperature,
                     const float* top_p, const int32_t* top_k, int32_t* main_out, int32_t* sem_code_out,
                     float* hidden_out, float* logits_out, void* stream);

/* Prefill ("Overall architecture & Dual-AR data flow", sections 3.1 and 4):
 * the prompt's positions n_past0 .. n_past0 + T - 1 run through the layers
 * of the step above causally, writing their keys and values into the cache;
 * the last position's logits give the first main token, drawn and checked
 * against the window exactly as s2fast_slow_step does.  The prompt runs in
 * chunks of up to 64 positions a launch on the matrix cores (one pass over
 * the weights a chunk; each position attends to the cache up to itself),
 * the last chunk holding the last position, whose head and draw then take
 * one short launch; when the last chunk would hold only the last position,
 * that position is a step launch of its own.  With an f32 cache the chunks
 * stop where a chunk's attention scores no longer fit on chip (several
 * thousand positions), and the rest runs two positions a launch (one
 * weight pass for both, the second attending to the first).  The pages'
 * engine takes one token per chunk on CUDA.
 *   tokens [T, 1 + num_codebooks] i32: per position the row-0 token (text,
 *          marker or semantic id), then the codebook codes; the codes count
 *          only where the row-0 token is a semantic id (the prompt's mask)
 * Other arguments as s2fast_slow_step.  The first call on a context that
 * runs chunks sets them up: it packs a second copy of the layer matrices
 * for the matrix cores (7.3 GB at the S2 Pro shape) and allocates their
 * arena, synchronising the device; later calls only enqueue.  Errors:
 * S2FAST_ERR_ARG for NULL pointers (other than logits_out), misaligned
 * kv_cache / hidden_out, T < 1 or positions outside [0, max_context);
 * S2FAST_ERR_NOMEM / S2FAST_ERR_HIP if that set-up fails (nothing is
 * enqueued, and later calls run two positions a launch).  Shapes the chunk
 * kernel cannot take run two positions a launch without a set-up. */
int s2fast_slow_prefill(s2fast_slow_ctx* ctx, void* kv_cache, int32_t n_past0, int32_t T, const int32_t* tokens,
                        int32_t* window, const float* u, const float* temperature, const float* top_p,
                        const int32_t* top_k, int32_t* main_out, int32_t* sem_code_out, float* hidden_out,
                        float* logits_out, void* stream);

/* One full frame ("Fast-AR codebook decoding ...", section 5.1): the Slow-AR
 * step above, then s2fast_decode_frame of one request on its hidden state
 * and semantic code.  The fast context must have in_dim == dim (else
 * S2FAST_ERR_HIDDEN_DIM, the pages' hidden-width check, section 1) and the
 * same codebook_size and num_codebooks (else S2FAST_ERR_ARG).
 *   u_slow [2], u_fast [num_codebooks-1] f32; main_out [1] i32 OUT;
 *   hidden_out [dim] f32 OUT (16-byte aligned); codes_out [num_codebooks]
 *   i32 OUT [sem_code, c_1, ..., c_9].
 * A following frame passes main_out and codes_out as prev_main and
 * prev_codes and n_past + 1; the caller stops at end_id.  If the Slow-AR
 * launch fails, S2FAST_ERR_HIP is returned and no output is written; a
 * failure of the Fast-AR part follows s2fast_decode_frame (codes_out[1:]
 * zero-filled). */
int s2fast_full_frame(s2fast_slow_ctx* slow, s2fast_ctx* fast, void* kv_cache, int32_t n_past,
                      const int32_t* prev_main, const int32_t* prev_codes, int32_t* window, const float* u_slow,
                      const float* u_fast, const float* temperature, const float* top_p, const int32_t* top_k,
                      int32_t* main_out, float* hidden_out, int32_t* codes_out, void* stream);

/* Grid-wide synchronisation points of one Slow-AR step (one per layer,
 * after its wo phase; the other phases hand over tagged values), and the
 * number of head rows (n_allowed); -1 on error. */
int s2fast_slow_syncs(const s2fast_slow_ctx* ctx);
int s2fast_slow_allowed(const s2fast_slow_ctx* ctx);

/* ---- test exports (used by the test suite; not part of the hot path) ---- */

/* Host-side: the RoPE table the context uses, [context, head_dim/2] cos and
 * sin as float32 holding bf16-rounded values of cos/sin(p * base^(-2i/hd))
 * (Mizuoto page, "What matches upstream").  cos_out / sin_out are HOST pointers. */
int s2fast_test_rope_table(int32_t head_dim, int32_t context, float rope_base,
                           float* cos_out, float* sin_out);

/* Streaming-read probe (the achievable HBM read rate the roofline quotes
 * beside the 8 TB/s specification): one launch of `grid` workgroups x 512
 * threads reads the `bytes` at `src` (device, 16-byte aligned, bytes a
 * multiple of 16) with 16-byte non-temporal loads, `in_flight` (4 or 8) a
 * thread, block b taking a contiguous 1/grid of the buffer, and writes the
 * XOR of every 32-bit word of the buffer to *sink (device; cleared first).
 * Enqueued on `stream`.  S2FAST_ERR_ARG for NULL or misaligned pointers,
 * a size of 0 or not a multiple of 16, grid outside [1, 65535] or another
 * in_flight; S2FAST_ERR_DEVICE off gfx950. */
int s2fast_test_stream_read(const void* src, uint64_t bytes, int32_t grid, int32_t in_flight, uint32_t* sink,
                            void* stream);

/* Device sampler on caller-supplied logits [B, V] (device), with the same
 * settings layout as s2fast_decode_frame but one uniform per request
 * (u [B]).  Writes codes [B] (device).  V <= 8192. */
int s2fast_test_sample(int32_t B, int32_t V, const float* logits, const float* temperature,
                       const float* top_p, const int32_t* top_k, const float* u, int32_t* codes,
                       void* stream);

/* The frame kernel's GEMV on its own (weight-streaming, 16-byte weight
 * loads, rows split over one block per CU), for per-kernel parity:
 *   y[m, :] = W . n_m  for m < M (M = 1 or 2),  n_m = x[m, :] * norm_w / rms(x[m, :])
 *   when norm_w is not NULL (RMSNorm, "Model loading and GGUF", section 2.2),
 *   else n_m = x[m, :]; with W3 not NULL the output is the SwiGLU pair
 *   silu(W . n_m) * (W3 . n_m) ("Fast-AR codebook decoding ...", section 3).
 *   W, W3 [N, K] of weight_dtype and norm_w [K] (bf16 for S2FAST_Q8, else
 *   weight_dtype); with S2FAST_Q8, scale / scale3 [N] f32 are the row scales
 *   of W / W3 (NULL otherwise); x [M, K] f32; y [M, N] f32 OUT; device
 *   pointers, W / W3 / x 16-byte aligned; K a multiple of 8 (bf16), 16
 *   (int8) or 4 (f32), K <= 16384.  Enqueued on `stream`.
 * Errors: S2FAST_ERR_ARG for bad sizes or pointers, S2FAST_ERR_DEVICE off
 * gfx950. */
int s2fast_test_gemv(int32_t weight_dtype, int32_t N, int32_t K, int32_t M, const void* W, const void* W3,
                     const float* scale, const float* scale3, const void* norm_w, float eps, const float* x, float* y,
                     void* stream);

/* The frame kernel's q/k RMSNorm + pair RoPE + causal attention (mask
 * offset 0) on its own ("Fast-AR codebook decoding ...", section 3; Mizuoto
 * page, "What matches upstream": bf16-rounded RoPE table): for every window
 * position t < T, the attention output of position t over positions 0..t.
 *   qkv    [T, (n_head + 2 n_head_kv) head_dim] f32: raw wqkv outputs
 *          (Q heads, K heads, V heads) of positions 0..T-1
 *   q_norm, k_norm [head_dim] f32, both NULL for no q/k norm
 *   out    [T, n_head head_dim] f32 OUT, heads in order
 * head_dim a multiple of 8 and <= 128; T <= context <= 16.  Device
 * pointers.  Blocking (it builds and uploads the RoPE table). */
int s2fast_test_norm_rope_attn(int32_t n_head, int32_t n_head_kv, int32_t head_dim, int32_t T, int32_t context,
                               float rope_base, float eps, const float* qkv, const float* q_norm,
                               const float* k_norm, float* out, void* stream);

/* Failure-path test hook: with give_up != 0, later launches on this
 * context make every block's first grid-wide wait target an epoch that no
 * block publishes and give up after its first polls, and every wait on
 * another block's tagged outputs (batch-1 frames, Slow-AR steps) give up at
 * once, so every block leaves the kernel normally and the failure path of
 * s2fast_status runs; 0 restores normal launches. */
int s2fast_test_watchdog(s2fast_ctx* ctx, int32_t give_up);
int s2fast_test_slow_watchdog(s2fast_slow_ctx* ctx, int32_t give_up);

/* Chunked-prefill switch: enable = 0 makes later s2fast_slow_prefill calls
 * on this context run every position two a launch (the comparison path);
 * 1 (the default) restores the chunks; enable = N > 1 keeps the chunks but
 * only below cache position N, as if the f32 cache's on-chip score buffer
 * ended there (the rest runs two positions a launch).  S2FAST_ERR_ARG for
 * a NULL context or enable < 0. */
int s2fast_test_slow_prefill_chunks(s2fast_slow_ctx* ctx, int32_t enable);

/* Timeline instrumentation (blocking; for measurement only).  enable != 0
 * makes later launches on this context record, for every block and every
 * record i < 256 of a frame (batch-1 launches: phase i; batched launches:
 * grid-wide synchronisation point i), the 100 MHz wall clock when the block
 * finished the phase (word 0) and when it left the synchronisation after it
 * (word 1: a grid sync, or the block's own barrier after a batch-1 phase
 * whose outputs the next phase waits on itself as tagged values); words
 * 2..7 hold in-phase marks (2: before the
 * GEMV, 3: after it, 4: input staged, 5: phase start, 6 and 7: after the
 * q/k norms and after the attention scores in the attention phase), 0 where
 * a phase sets none.  If host_out is not NULL (HOST pointer, capacity >= n_blocks*256*8
 * words) the device is synchronised and the last frame's record is copied
 * out as [block][i][8].  The buffer is allocated on the first call. */
int s2fast_test_timeline(s2fast_ctx* ctx, int32_t enable, uint32_t* host_out, int32_t capacity);

/* The same instrumentation for Slow-AR step launches (record i: phase i < 256
 * of a step, five a layer, then the head). */
int s2fast_test_slow_timeline(s2fast_slow_ctx* ctx, int32_t enable, uint32_t* host_out, int32_t capacity);

/* Number of grid-wide synchronisation points one frame of B requests
 * takes on this context, or -1 on error (for measurement reports).  A
 * batch-1 frame syncs after fast_project_in and after each layer's
 * attention + wo phase only. */
int s2fast_syncs_per_frame(const s2fast_ctx* ctx, int32_t B);

#ifdef __cplusplus
}
#endif

#endif /* S2FAST_H */
