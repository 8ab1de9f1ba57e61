/*
 * lmdecode.h - C ABI of the MI355X (gfx950) batch-1 decode step of a
 * Llama-architecture transformer with block-quantised weights.
 *
 * What one decode step computes (per sequence s, token t at position p):
 *   x = E[t]                                   fp16 embedding row -> fp32
 *   for each layer:
 *     xn = x / sqrt(mean(x^2) + eps) * g_attn  RMSNorm
 *     q, k, v = W_q xn, W_k xn, W_v xn         dequant-GEMV over Q8_0/Q4_0 blocks
 *     rotate q, k by RoPE at p; K[p] = fp16(k), V[p] = fp16(v)
 *     o_h = softmax_t(q_h . K[g][t] / sqrt(hd)) V[g][t], t = 0..p, g = h / (nq/nkv)
 *     x += W_o o
 *     xn = RMSNorm(x) * g_ffn;  x += W_down (silu(W_gate xn) * (W_up xn))
 *   logits = W_lm (RMSNorm(x) * g_out);  next token = argmax (lowest index on ties)
 * Sources: the C/CUDA Llama engine page (rskf.cn/news/15116) lists the Llama
 * features and the Q8_0/Q4_0 formats in section 1 and the operators in
 * section 4.4 (GEMV for single-token products, fused RMSNorm, RoPE from a
 * precomputed sin/cos table, SwiGLU fused with the FC product, causal-masked
 * softmax); the SwarmKV page ("Prefill once, fan out", ideipro.ru) gives the
 * KV size in section 3 and positions that continue after the prefix in
 * section 4; the weight-streaming mode follows the double-buffered pipeline
 * of the same engine page (sections 2.3, 3.3, 4.2) and the pinned-host /
 * two-stream / ping-pong-buffer design of "3 Agents. 3 LLMs. 1 Aging GPU"
 * (section on loading only the layers you need).
 *
 * Conventions for every call:
 *   - Host pointers passed in are read during the call only; the library
 *     copies what it keeps.  Device pointers (the *_dev call) stay owned by
 *     the caller.
 *   - The library owns all device memory (weights, KV cache, scratch, the two
 *     streaming buffers) and the pinned host arena of streaming mode.
 *   - No C++ exception crosses this boundary.  Every call returns a status;
 *     lm_last_error() returns a message with the numbers involved.
 *   - All-or-nothing: a failed call leaves the model as it was, and a failed
 *     lm_model_create leaks nothing.
 *   - A model is not thread-safe: the caller serialises calls on one model.
 *     Different models (on different streams) are independent.
 */
#ifndef LMDECODE_H
#define LMDECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lm_model lm_model;

typedef enum {
    LM_OK = 0,
    LM_E_ARG = 1,    /* invalid argument (shape, index, null pointer, size) */
    LM_E_STATE = 2,  /* call not legal in the model's current state */
    LM_E_OOM = 3,    /* device or pinned-host allocation failed */
    LM_E_HIP = 4,    /* a HIP runtime call failed (message names it) */
    LM_E_CTX = 5     /* the step would run past max_ctx */
} lm_status;

/* GGUF type ids of the block formats (the C/CUDA Llama engine page, section 1,
 * lists Q4_0, Q8_0, Q4_K, Q5_K and Q6_K among the formats it reads; the K formats
 * carry its 70B figures).
 * Q8_0: 34-byte block = fp16 d (little endian) + 32 int8 q; w = d * q.
 * Q4_0: 18-byte block = fp16 d + 16 bytes; byte j holds element j in its low
 *       nibble and element j+16 in its high nibble; w = (nibble - 8) * d.
 * Q4_K: 144-byte super-block of 256 weights (GGUF's published layout) = fp16
 *       d, fp16 dmin, 12 bytes packing a 6-bit scale sc_j and a 6-bit min m_j
 *       per 32-weight sub-block j, 128 bytes of nibbles (32-byte group g:
 *       sub-block 2g in the low nibbles, 2g+1 in the high ones);
 *       w = d * sc_j * q - dmin * m_j.
 * Q5_K: 176-byte super-block = the Q4_K header (d, dmin, 12 bytes of 6-bit
 *       pairs), 32 bytes of fifth bits (bit j of byte l: element 32j + l), 128
 *       bytes of low nibbles grouped as in Q4_K; w = d * sc_j * q - dmin * m_j,
 *       q = 5 bits.
 * Q6_K: 210-byte super-block of 256 weights = 128 bytes of low nibbles, 64
 *       bytes of 2-bit high parts, 16 int8 scales (one per 16 weights), fp16
 *       d; w = d * scale * (q - 32), q = 6 bits.
 * The K formats need every matrix input width (hidden, ffn, n_heads *
 * head_dim) to be a multiple of 256 and decode one sequence per step
 * (max_seqs = 1). */
typedef enum { LM_Q4_0 = 2, LM_Q8_0 = 8, LM_Q4_K = 12, LM_Q5_K = 13, LM_Q6_K = 14 } lm_qtype;

typedef struct {
    int32_t vocab;       /* rows of the LM head, rows of the embedding table; even and >= 2
                            (the GEMV finishes its rows in adjacent pairs) */
    int32_t hidden;      /* H, a multiple of 32 */
    int32_t n_layers;
    int32_t n_heads;     /* query heads nq */
    int32_t n_kv_heads;  /* KV heads nkv; nq % nkv == 0, nq / nkv <= 8 */
    int32_t head_dim;    /* hd: 64 or 128 */
    int32_t ffn;         /* F, a multiple of 32 */
    double rms_eps;      /* RMSNorm epsilon (inside the square root) */
    double rope_theta;   /* RoPE base: pair i turns by p * theta^(-2i/hd) */
    int32_t max_ctx;     /* KV positions per sequence */
    int32_t max_seqs;    /* sequences decoded together (1..4; 2..4 need hidden <= 6144) */
    int32_t qtype;       /* an lm_qtype, for every weight matrix (the LM head included) */
} lm_config;

/* One decoder layer's weights.  Norm gains: fp32 [hidden].  Matrices: GGUF
 * block bytes, row-major [out rows][in/32 blocks] (in/256 super-blocks for
 * the K formats):
 *   wq [nq*hd][H], wk [nkv*hd][H], wv [nkv*hd][H], wo [H][nq*hd],
 *   w_gate [F][H], w_up [F][H], w_down [H][F]. */
typedef struct {
    const float* attn_norm;
    const float* ffn_norm;
    const void* wq;
    const void* wk;
    const void* wv;
    const void* wo;
    const void* w_gate;
    const void* w_up;
    const void* w_down;
} lm_layer_weights;

/* Validates cfg, then allocates every device buffer the model needs (KV
 * cache for max_seqs x max_ctx, weights, scratch).  The KV cache holds
 * n_layers x n_kv_heads x max_ctx x head_dim x 2 (K and V) fp16 values per
 * sequence, the size the SwarmKV page ("Prefill once, fan out", section 3)
 * gives; the model shapes are the Llama features of the C/CUDA Llama engine
 * page (section 1: RoPE, GQA, SwiGLU, RMSNorm).  hip_stream: a hipStream_t
 * the model launches on (borrowed, never destroyed), or NULL for a stream the
 * library creates.  On failure *out is NULL and nothing is left allocated.
 * Errors: LM_E_ARG (bad config, with the offending field), LM_E_OOM, LM_E_HIP. */
lm_status lm_model_create(const lm_config* cfg, void* hip_stream, lm_model** out);

/* Waits for the model's work, then frees everything it owns.  NULL is a no-op. */
void lm_model_destroy(lm_model* m);

/* Copies one layer's weights (host memory) into the model, repacking the
 * blocks into the library's device layout.  The blocks are GGUF's (the C/CUDA
 * Llama engine page, section 1, reads GGUF files in these formats); byte
 * counts follow from the config.  Errors: LM_E_ARG (layer out of range, NULL
 * pointer), LM_E_OOM, LM_E_HIP. */
lm_status lm_load_layer_weights(lm_model* m, int32_t layer, const lm_layer_weights* w);

/* Embedding table fp16 bits [vocab][hidden], output norm gain fp32 [hidden],
 * LM head GGUF blocks [vocab][hidden/32].  The model is ready to decode once
 * this and every layer are loaded. */
lm_status lm_load_global_weights(lm_model* m, const uint16_t* tok_embd_f16,
                                 const float* out_norm, const void* lm_head_blocks);

/* Installs n_pos cached (already rotated) keys and values of one (sequence,
 * layer): fp16 bits [n_kv][n_pos][head_dim] each.  Sets the sequence's next
 * position to n_pos (its next decode step runs at position n_pos, 0-based).
 * Errors: LM_E_ARG (index or n_pos > max_ctx), LM_E_HIP. */
lm_status lm_load_kv(lm_model* m, int32_t seq, int32_t layer, const uint16_t* k,
                     const uint16_t* v, int32_t n_pos);

/* Copies cached rows 0..n_pos-1 of one (sequence, layer) out, same layout. */
lm_status lm_get_kv(lm_model* m, int32_t seq, int32_t layer, uint16_t* k, uint16_t* v,
                    int32_t n_pos);

/* Rewinds (or advances) a sequence: its next step runs at position pos and
 * overwrites cache rows >= pos. 0 <= pos <= max_ctx. */
lm_status lm_set_position(lm_model* m, int32_t seq, int32_t pos);
lm_status lm_get_position(const lm_model* m, int32_t seq, int32_t* pos);

/* Weight residency (the C/CUDA Llama engine page's tiered layer cache, its
 * sections 2.2-2.3, 3.2-3.3 and 4.1-4.2: tier A in GPU memory, tier B in pinned
 * host memory streamed through two GPU layer buffers).  Layers
 * 0..n_resident-1 stay in HBM; layers n_resident..L-1 move to a pinned host
 * arena, and each step copies streamed layer l+1 into one of two HBM layer
 * buffers on a copy stream while layer l computes from the other (events order
 * both the copy->compute and the compute->overwrite edges; the next step's
 * first two streamed layers are copied while the LM head runs).  n_resident = L:
 * everything resident (the state after lm_model_create); 0: every layer
 * streamed.  Embedding, norms, LM head and KV stay in HBM always.  Legal only
 * between steps; the weights move (device memory peaks at old + new resident
 * arenas).  The pinned arena is kept when it can hold the new streamed set
 * (more layers resident, or fewer when the front it freed before is large
 * enough; that front stays allocated until the arena is replaced); otherwise a
 * new one is allocated before the old one is freed.  Outputs are
 * bit-identical for every n_resident.
 * Errors: LM_E_ARG (n_resident outside 0..L), LM_E_OOM (pinned or device
 * memory; the model is unchanged), LM_E_HIP. */
lm_status lm_set_residency(lm_model* m, int32_t n_resident);

/* Layer skip (the C/CUDA Llama engine page, sections 2.5, 3.5 and 4.5: a
 * layer whose output is close to its input is skipped; section 3.5 calibrates
 * which).  mask: host uint8 [n_layers], nonzero = skip the layer; NULL clears
 * the mask.  A skipped layer computes nothing and writes no KV-cache row: its
 * input is its output.  In streaming mode skipped layers are not copied.
 * Changing the mask mid-sequence leaves the skipped steps' cache rows of
 * those layers unwritten.  Legal only between steps.  Errors: LM_E_HIP. */
lm_status lm_set_layer_skip(lm_model* m, const uint8_t* mask);

/* Similarity recording for calibrating the skip list.  enable = 1 clears the
 * accumulators; every following step (run without graphs) adds, for each
 * computed layer and sequence, the cosine similarity a.b / (|a| |b|) of the
 * layer's input and output hidden vectors (fp64; 0 when either is zero).
 * enable = 0 stops recording and keeps the sums.  Errors: LM_E_HIP. */
lm_status lm_layer_similarity(lm_model* m, int32_t enable);

/* mean: host fp64 [n_layers], the recorded similarities' mean per layer (NaN
 * for a layer with no record); count: host int32 [n_layers] records, or NULL.
 * Synchronises the model's stream.  Errors: LM_E_ARG (NULL mean), LM_E_HIP. */
lm_status lm_get_layer_similarity(lm_model* m, double* mean, int32_t* count);

/* The calibrated skip list: skips exactly the layers whose recorded mean
 * similarity is above threshold (the page's default is 0.98) and reports how
 * many in *n_skipped (nullable); lm_set_layer_skip with that mask.
 * Errors: LM_E_ARG (non-finite threshold), LM_E_HIP. */
lm_status lm_skip_similar_layers(lm_model* m, double threshold, int32_t* n_skipped);

/* One self-speculative round for sequence 0 (the C/CUDA Llama engine page,
 * sections 3.5 and 5.3: draft with the bottom layers, verify with the full
 * model).  token: sequence 0's next input token (at its position p, not yet
 * processed).  k drafts d1..dk, each a step through layers 0..draft_layers-1
 * and the LM head; then one pass of every layer over t0 = token, d1..dk at
 * positions p..p+k (k+1 columns of the several-sequence path, all on sequence
 * 0's cache, so column j attends to keys 0..p+j: the same as k+1 plain
 * steps); then the longest prefix of drafts the full model agrees with, plus
 * the full model's own token after it, go to tokens_out (host int32 [k+1]),
 * their count to *n_out (1..k+1) and sequence 0's position becomes
 * p + *n_out; the last output token is the next round's input.  Greedy
 * decoding gives the same tokens.  Cache rows past the new position hold
 * draft or rejected values until overwritten.  Needs 1 <= k <= 3, k + 1 <=
 * max_seqs, every layer resident.  Blocks until the tokens are on the host.
 * Errors: LM_E_ARG, LM_E_STATE (weights not loaded, streaming mode, a model
 * created for one sequence - the K formats are), LM_E_CTX (p + k + 1 >
 * max_ctx), LM_E_HIP. */
lm_status lm_speculative_step(lm_model* m, int32_t token, int32_t draft_layers, int32_t k,
                              int32_t* tokens_out, int32_t* n_out);

/* 0: every layer resident (lm_set_residency(m, L)); 1: every layer streamed
 * (lm_set_residency(m, 0)), each layer's copy overlapping the compute of the
 * layers before it; 2: every layer streamed serially, as the baseline of the
 * two-buffer pipeline of the "3 Agents" page's layer-loading section: a
 * layer's copy starts only when every kernel before it has finished, and its
 * kernels wait for it (copy, compute, copy, compute).  Outputs are the same
 * in every mode.  Errors: those of lm_set_residency; LM_E_ARG (mode). */
lm_status lm_stream_mode(lm_model* m, int32_t enable);

/* The engine page's tier sizing (its section 4.1, compute_tier_sizes):
 * tier_a = min(L, floor(0.9 * hbm_bytes / layer_bytes)) layers in HBM, then
 * tier_b = min(L - tier_a, floor(0.7 * host_bytes / layer_bytes)) in pinned
 * host memory.  Pure host arithmetic (no device needed).
 * Returns LM_OK when tier_a + tier_b == n_layers, LM_E_OOM when layers are
 * left over (the pages' disk tier, which this library does not have),
 * LM_E_ARG on a NULL output or a non-positive size. */
lm_status lm_tier_sizes(int32_t n_layers, int64_t layer_bytes, int64_t hbm_bytes, int64_t host_bytes,
                        int32_t* tier_a, int32_t* tier_b);

/* lm_tier_sizes for this model's layer blobs: hbm_bytes <= 0 means the
 * device's free memory now plus what the resident layers hold; host_bytes <= 0
 * the host's available memory plus what the host arena holds.  *n_resident =
 * tier A, ready for lm_set_residency.  Errors: LM_E_OOM (the rest does not fit
 * in host memory; *n_resident is still set), LM_E_HIP. */
lm_status lm_plan_residency(lm_model* m, int64_t hbm_bytes, int64_t host_bytes, int32_t* n_resident);

/* One decode step for sequences 0..n_seq-1 (1 <= n_seq <= max_seqs): the
 * operator chain at the top of this file, i.e. the C/CUDA Llama engine page's
 * section 4.4 operators (single-token GEMV, fused RMSNorm, RoPE from a
 * precomputed table, causal-masked softmax attention, SwiGLU fused with the FC
 * product) over the model of its section 1, each sequence at its own position
 * (positions continue after the cached prefix: the SwarmKV page, section 4).
 * tokens host int32 [n_seq]; logits host fp32 [n_seq][vocab] or NULL;
 * argmax host int32 [n_seq].  Blocks until the results are on the host.
 * Every sequence advances by one position.
 * Errors: LM_E_STATE (weights not all loaded), LM_E_ARG (token out of range,
 * n_seq out of range), LM_E_CTX (a sequence at max_ctx; checked before any
 * device work), LM_E_HIP. */
lm_status lm_decode_step(lm_model* m, const int32_t* tokens, int32_t n_seq, float* logits,
                         int32_t* argmax);

/* The same step on device buffers, asynchronous on the model's stream:
 * d_tokens int32 [n_seq], d_logits fp32 [n_seq][vocab] or NULL, d_argmax int32
 * [n_seq].  Token ids are not range-checked on the host (the kernel clamps an
 * out-of-range id to 0).  d_argmax may equal d_tokens to feed the greedy loop
 * on the device. */
lm_status lm_decode_step_dev(lm_model* m, const int32_t* d_tokens, int32_t n_seq,
                             float* d_logits, int32_t* d_argmax);

/* lm_decode_step_dev for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results; it calls no hipMalloc,
 * hipFree or allocating routine and instantiates no graph (its kernels are
 * launched one by one on the model's stream, so a caller may capture them).
 * The step's working memory (residual, q, attention output, FFN hidden,
 * activation digits, attention partial states and counts, argmax candidates
 * and counts) lives in a fixed 32 MiB device array inside the library, one
 * per GPU, held until the process ends.  Each call clears the counts it
 * uses; every call on a GPU shares that GPU's array, so calls that overlap on
 * one GPU (two streams, two threads) race and must be serialised by the
 * caller.  Errors: those of lm_decode_step_dev; LM_E_ARG when n_seq
 * sequences at this model's max_ctx need more than the array holds (the
 * attention partial states grow with n_seq * n_heads * max_ctx; the message
 * gives the size); LM_E_STATE when a layer is streamed (every layer must be
 * resident). */
lm_status lm_decode_step_dev_noalloc(lm_model* m, const int32_t* d_tokens, int32_t n_seq,
                                     float* d_logits, int32_t* d_argmax);

/* 1 (default): replay each step from a captured HIP graph; 0: launch eagerly. */
lm_status lm_set_graph(lm_model* m, int32_t enable);

/* The hipStream_t the model launches on. */
void* lm_stream(const lm_model* m);

/* Last error message of this model, or of the calling thread's last failed
 * lm_model_create when m is NULL.  Never NULL; "" when there is none. */
const char* lm_last_error(const lm_model* m);

/* ---- measurement and inspection ---------------------------------------- */

/* Kernel families of one step (for timing and profiling).  LM_K_COPY is the
 * host-to-HBM copy of one layer blob on the copy stream in streaming mode
 * (its durations are those copies' events; its bytes are the blobs copied per
 * step, zero when the weights are resident). */
typedef enum {
    LM_K_EMBED = 0, LM_K_QKV = 1, LM_K_ATTN = 2, LM_K_WO = 3, LM_K_GATEUP = 4,
    LM_K_DOWN = 5, LM_K_LMHEAD = 6, LM_K_COPY = 7, LM_K_COUNT = 8
} lm_kernel_kind;

/* enable = 1: eager steps record HIP events around every kernel of every
 * kind on the model's stream (and around every layer copy on the copy stream
 * in streaming mode) and accumulate their durations; graph replay is
 * suspended.  enable = 2: the same events are captured into the step's HIP
 * graph (event-record nodes beside the kernels), and every replay waits for
 * the step and accumulates them - kernel times as the replayed step runs them
 * (streaming mode, which does not replay graphs, times eagerly).  0: off.
 * Resets the totals; changing the mode drops captured graphs. */
lm_status lm_kernel_timing(lm_model* m, int32_t enable);

/* Average duration of one launch of kernel family `kind` as the step graph
 * runs it: the step's launches of that family alone (same arguments and
 * order; an LM-head-only replay does not advance positions) are captured as
 * one graph (a family launched once per step: 32 copies of it) and replayed
 * `reps` times between two HIP events on the model's stream; result =
 * elapsed / (reps x the launches in the graph).  It
 * overwrites activations
 * and the current position's K/V row like a step (the next step rewrites
 * them).  Resident weights only.  For the roofline of a kernel family. */
lm_status lm_time_kind(lm_model* m, int32_t kind, int32_t n_seq, int32_t reps, double* us_per_launch);

/* Launch count and summed duration (ms) of one kernel kind since timing was
 * enabled (events are read after the step's final synchronisation). */
lm_status lm_kernel_stats(lm_model* m, int32_t kind, int64_t* count, double* total_ms);

/* Algorithmic bytes one launch of `kind` moves (weights + activations + KV,
 * at the sequences' current positions for attention), summed over the
 * launches of one step. */
lm_status lm_kernel_bytes(const lm_model* m, int32_t kind, int32_t n_seq, double* bytes);

/* Dequantises rows [row0, row0 + n_rows) of one loaded matrix with a GPU
 * kernel that reads the library's device layout, into host fp32 [n_rows][cols].
 * which: 0 wq, 1 wk, 2 wv, 3 wo, 4 w_gate, 5 w_up, 6 w_down (layer >= 0) or
 * 7 the LM head (layer ignored).  Values are exact (d * q fits fp32). */
lm_status lm_debug_dequant(lm_model* m, int32_t layer, int32_t which, int32_t row0,
                           int32_t n_rows, float* out);

/* The step's dequant-GEMV kernel on a given input: y = W x with no RMSNorm
 * gain and no epilogue (W from a resident layer, or the LM head).  which: 0
 * the QKV matrix (rows: the nq*hd query rows, then nkv*hd key rows, then
 * nkv*hd value rows; input hidden), 1 Wo (input nq*hd), 2 gate/up (row 2i =
 * gate row i, row 2i+1 = up row i; input hidden), 3 down (input ffn), 4 the LM
 * head (layer ignored).  x: host fp32 [n_seq][K]; y: host fp32 [n_seq][N].
 * n_seq = 1 runs the one-sequence kernel, 2..max_seqs the matrix-core path.
 * It allocates and frees a device buffer of its own.  For checking the
 * products against a reference.  Errors: LM_E_ARG, LM_E_STATE (the layer is
 * streamed), LM_E_HIP. */
lm_status lm_debug_gemv(lm_model* m, int32_t layer, int32_t which, int32_t n_seq, const float* x,
                        float* y);

/* Fault injection for the all-or-nothing contract: the n-th device or
 * pinned-host allocation the library makes from now on (in any model of the
 * process) fails as if memory were exhausted (LM_E_OOM); n <= 0 disarms it.
 * lm_debug_alloc_count: the number of allocations the library has attempted
 * in this process. */
void lm_debug_fail_alloc(int64_t n);
int64_t lm_debug_alloc_count(void);

/* A read-only kernel over n_bytes of device memory (sum of 16-byte words,
 * with the non-temporal loads the GEMVs read their weights with), for
 * calibrating HBM counters and the read ceiling; *ms = average duration over
 * iters launches. */
lm_status lm_debug_read_bw(lm_model* m, int64_t n_bytes, int32_t iters, double* ms);

#ifdef __cplusplus
}
#endif

#endif /* LMDECODE_H */
