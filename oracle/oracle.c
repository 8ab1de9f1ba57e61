/*
 * oracle.c - plain, slow fp64 CPU oracle of the batch-1 decode step of a
 * Llama-architecture transformer with block-quantised (Q8_0 / Q4_0) weights.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this code.  The product path (the HIP library)
 * never links, loads or calls it, and this file shares no header, helper,
 * table or constant generator with that library.
 *
 * Every step is the plain definition written out in fp64, one output element
 * at a time; OpenMP only spreads independent output rows over threads.  No
 * blocking, no fusion, no reordering of a definition's terms beyond what the
 * definition states.
 *
 * Sources (the pages' titles; section numbers are the pages' own):
 *   [ENGINE]  "pure C + CUDA Llama inference engine" (rskf.cn/news/15116):
 *             section 1 lists the Llama features (RoPE, GQA, SwiGLU, RMSNorm,
 *             KV cache) and the GGUF block formats (Q4_0, Q8_0); section 4.4
 *             lists the operators: GEMV for the single-token vector-matrix
 *             product, RMSNorm with its scale, RoPE from a precomputed sin/cos
 *             table, SwiGLU fused with the fully connected product, softmax
 *             with the causal mask.
 *   [SWARMKV] "Prefill once, fan out: KV snapshots for multi-agent LLM
 *             pipelines" (ideipro.ru): section 3 (problem A) gives the KV
 *             cache size n_layers * n_head_kv * n_ctx * head_dim * dtype * 2;
 *             section 4 step 4 says decode positions continue from the end of
 *             the prefix, or RoPE goes wrong.
 *   [ENGINE] sections 3.5 and 5.3 (self-speculative decoding): the bottom
 *             layers draft tokens, the full model verifies them.
 *   [ENGINE] sections 2.5, 3.5 and 4.5 (layer skip): a layer whose output is
 *             close to its input, by the cosine similarity of the two hidden
 *             vectors against a threshold (0.98 by default), is skipped and its
 *             input passed on; section 3.5 calibrates the similarities ahead
 *             of time.
 * The block formats are the ones the workload states: Q8_0 = fp16 d then 32
 * int8 q, value d*q; Q4_0 = fp16 d then 16 bytes, byte j = element j (low
 * nibble) | element j+16 (high nibble), value (nibble - 8) * d.
 * [ENGINE] section 1 also names the GGUF "K" formats Q4_K and Q6_K (the
 * formats of its 70B figures) without defining them; their byte layout is the
 * one the GGUF format publishes (restated in orc_dequant_row below): 256-weight
 * super-blocks,
 *   Q4_K (144 bytes): fp16 d, fp16 dmin, 12 bytes packing eight 6-bit scales
 *         sc_j and eight 6-bit mins m_j (one per 32-weight sub-block j), then
 *         128 bytes of nibbles; value d*sc_j*q - dmin*m_j, q in 0..15;
 *   Q5_K (176 bytes): the Q4_K header (fp16 d, fp16 dmin, 12 bytes of 6-bit
 *         scale/min pairs), 32 bytes of high bits (byte l, bit j: element
 *         32j + l), 128 bytes of low nibbles grouped as in Q4_K; value
 *         d*sc_j*q - dmin*m_j, q in 0..31;
 *   Q6_K (210 bytes): 128 bytes of low nibbles, 64 bytes of 2-bit high parts,
 *         16 int8 scales (one per 16-weight sub-block), fp16 d; value
 *         d*scale*(q - 32), q in 0..63.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   RoPE rotates adjacent pairs (2i, 2i+1) by angle pos * theta^(-2i/hd), no
 *   frequency scaling; the cached prefix keys are already rotated; positions
 *   are 0-based and the first decode token of a sequence with n cached
 *   entries sits at position n; the new token's k and v are rounded to fp16
 *   (nearest even) into the cache before attention reads them; attention
 *   scale 1/sqrt(hd), keys 0..pos inclusive; query head h reads KV head
 *   floor(h / (n_heads / n_kv_heads)); RMSNorm x / sqrt(mean(x^2) + eps) * g;
 *   no biases; the LM head is its own quantised matrix; argmax picks the
 *   first index of the largest fp32-rounded logit.  Layer skip: a skipped
 *   layer computes nothing and writes no cache row (its input is its output);
 *   a layer's similarity is the cosine of its input and output residual
 *   vectors (0 when either is zero); the calibrated list skips a layer when
 *   its similarity, averaged over the calibration steps and sequences, is
 *   above the threshold.
 *
 * parity pins: see tests/test_oracle_pins.py (every function here has one).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_Q4_0 2
#define ORC_Q8_0 8
#define ORC_Q4_K 12
#define ORC_Q5_K 13
#define ORC_Q6_K 14

/* ------------------------------------------------------------------------ */
/* IEEE binary16 <-> fp64                                                    */
/* ------------------------------------------------------------------------ */

/* Exact value of an IEEE binary16 bit pattern (subnormals kept). */
double orc_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0) v = ldexp((double)m, -24);                 /* subnormal / zero */
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);            /* (1 + m/1024) 2^(e-15) */
    return sign ? -v : v;
}

/* Round an fp64 value to binary16, nearest with ties to even. Works on the
 * fp64 bit pattern: keep 10 fraction bits, round on the dropped ones. */
uint16_t orc_f64_to_f16(double v) {
    uint64_t b;
    memcpy(&b, &v, 8);
    uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
    int e64 = (int)((b >> 52) & 0x7FF);
    uint64_t frac = b & 0xFFFFFFFFFFFFFull;
    if (e64 == 0x7FF) return (uint16_t)(sign | (frac ? 0x7E00u : 0x7C00u));
    if (e64 == 0) return sign;                              /* fp64 zero / tiny subnormal */
    int e = e64 - 1023;                                     /* v = 1.frac * 2^e */
    uint64_t sig = frac | (1ull << 52);                     /* 53-bit significand */
    int shift;                                              /* bits to drop */
    uint16_t exp_field;
    if (e >= -14) { shift = 42; exp_field = (uint16_t)(e + 15); }
    else {                                                  /* fp16 subnormal range */
        shift = 42 + (-14 - e);
        exp_field = 0;
        if (shift > 63) return sign;
    }
    uint64_t kept = sig >> shift;
    uint64_t rem = sig & ((1ull << shift) - 1);
    uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (kept & 1))) kept += 1;
    /* kept includes the hidden bit in the normal case */
    uint32_t out;
    if (exp_field == 0) out = (uint32_t)kept;               /* 1024 carries into exponent 1 */
    else {
        if (kept >= 2048) { kept >>= 1; exp_field += 1; }
        if (exp_field >= 31) return (uint16_t)(sign | 0x7C00u);
        out = ((uint32_t)exp_field << 10) | (uint32_t)(kept & 0x3FF);
    }
    return (uint16_t)(sign | out);
}

/* ------------------------------------------------------------------------ */
/* dequantisation (the formats the workload defines; [ENGINE] section 1)     */
/* ------------------------------------------------------------------------ */

int orc_block_bytes(int qtype) {
    switch (qtype) {
        case ORC_Q8_0: return 34;
        case ORC_Q4_0: return 18;
        case ORC_Q4_K: return 144;
        case ORC_Q5_K: return 176;
        case ORC_Q6_K: return 210;
        default: return -1;
    }
}

/* weights per block: 32 (Q8_0, Q4_0) or 256 (the K formats' super-blocks) */
int orc_block_weights(int qtype) {
    return qtype == ORC_Q4_K || qtype == ORC_Q5_K || qtype == ORC_Q6_K ? 256 : 32;
}

/* bytes of one row of `cols` weights, or -1 for an unknown type or a ragged row */
int64_t orc_row_bytes(int qtype, int64_t cols) {
    int bb = orc_block_bytes(qtype), qk = orc_block_weights(qtype);
    if (bb < 0 || cols % qk) return -1;
    return cols / qk * bb;
}

/* Q4_K: the 6-bit scale and min of sub-block j (0..7) from the 12 packed
 * bytes.  Sub-blocks 0..3 keep theirs in the low 6 bits of bytes j (scale) and
 * j+4 (min); sub-blocks 4..7 keep the low 4 bits of each in byte j+4 (scale in
 * the low nibble, min in the high one) and the top 2 bits in the spare top
 * bits of bytes j-4 (scale) and j (min). */
static void q4k_scale_min(const uint8_t* s, int j, int* sc, int* mn) {
    if (j < 4) {
        *sc = s[j] & 63;
        *mn = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *mn = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* One row of `cols` weights stored as consecutive blocks -> fp64 (exact). */
int orc_dequant_row(int qtype, const uint8_t* row, int64_t cols, double* out) {
    const int bb = orc_block_bytes(qtype), qk = orc_block_weights(qtype);
    if (bb < 0 || cols % qk) return -1;
    for (int64_t b = 0; b < cols / qk; ++b) {
        const uint8_t* blk = row + b * bb;
        double* o = out + qk * b;
        if (qtype == ORC_Q8_0) {
            double d = orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
            for (int j = 0; j < 32; ++j) o[j] = d * (double)(int8_t)blk[2 + j];
        } else if (qtype == ORC_Q4_0) {
            double d = orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
            for (int j = 0; j < 16; ++j) {
                int lo = blk[2 + j] & 0x0F, hi = blk[2 + j] >> 4;
                o[j] = (double)(lo - 8) * d;
                o[j + 16] = (double)(hi - 8) * d;
            }
        } else if (qtype == ORC_Q4_K) {
            /* element e of the super-block: sub-block j = e / 32; the 32 bytes
             * 32*(j/2) .. +31 of the nibble area hold sub-blocks j (even: low
             * nibbles) and j+1 (odd: high nibbles), element e at byte e % 32 */
            double d = orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
            double dmin = orc_f16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
            const uint8_t* scales = blk + 4;
            const uint8_t* qs = blk + 16;
            for (int e = 0; e < 256; ++e) {
                int j = e / 32, sc, mn;
                q4k_scale_min(scales, j, &sc, &mn);
                uint8_t byte = qs[32 * (j / 2) + e % 32];
                int q = (j % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
                o[e] = d * (double)sc * (double)q - dmin * (double)mn;
            }
        } else if (qtype == ORC_Q5_K) {
            /* as Q4_K, the nibble area after 32 bytes of high bits: element e
             * of sub-block j = e / 32 takes bit j of high-bit byte e % 32 as
             * its fifth bit */
            double d = orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
            double dmin = orc_f16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
            const uint8_t* scales = blk + 4;
            const uint8_t* qh = blk + 16;
            const uint8_t* qs = blk + 48;
            for (int e = 0; e < 256; ++e) {
                int j = e / 32, sc, mn;
                q4k_scale_min(scales, j, &sc, &mn);
                uint8_t byte = qs[32 * (j / 2) + e % 32];
                int q = ((j % 2 == 0) ? (byte & 0x0F) : (byte >> 4)) | (((qh[e % 32] >> j) & 1) << 4);
                o[e] = d * (double)sc * (double)q - dmin * (double)mn;
            }
        } else {  /* ORC_Q6_K */
            /* element e: half h = e / 128, r = e % 128, quarter t = r / 32,
             * l = r % 32.  Low 4 bits: byte 64h + l + 32*(t % 2), low nibble
             * for t < 2, high nibble for t >= 2.  High 2 bits: bits 2t, 2t+1 of
             * byte 32h + l of the high-bit area.  Scale: int8 number e / 16. */
            const uint8_t* ql = blk;
            const uint8_t* qh = blk + 128;
            const int8_t* scales = (const int8_t*)(blk + 192);
            double d = orc_f16_to_f64((uint16_t)(blk[208] | (blk[209] << 8)));
            for (int e = 0; e < 256; ++e) {
                int h = e / 128, r = e % 128, t = r / 32, l = r % 32;
                uint8_t lb = ql[64 * h + l + 32 * (t % 2)];
                int lo = t < 2 ? (lb & 0x0F) : (lb >> 4);
                int hi = (qh[32 * h + l] >> (2 * t)) & 3;
                int q = lo | (hi << 4);
                o[e] = d * (double)scales[e / 16] * (double)(q - 32);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* matrix-vector product over quantised rows ([ENGINE] section 4.4, GEMV)    */
/* y[r] = sum_c W[r][c] * x[c], W dequantised exactly, summed in order of c. */
/* ------------------------------------------------------------------------ */
int orc_gemv(int qtype, const uint8_t* w, int64_t rows, int64_t cols, const double* x, double* y) {
    const int64_t row_bytes = orc_row_bytes(qtype, cols);
    if (row_bytes < 0) return -1;
    #pragma omp parallel
    {
        double* wr = (double*)malloc(sizeof(double) * (size_t)cols);
        #pragma omp for schedule(static)
        for (int64_t r = 0; r < rows; ++r) {
            orc_dequant_row(qtype, w + r * row_bytes, cols, wr);
            double acc = 0.0;
            for (int64_t c = 0; c < cols; ++c) acc += wr[c] * x[c];
            y[r] = acc;
        }
        free(wr);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* RMSNorm ([ENGINE] sections 1 and 4.4): out = x / sqrt(mean(x^2) + eps) * g */
/* ------------------------------------------------------------------------ */
void orc_rmsnorm(const double* x, const float* g, int64_t n, double eps, double* out) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int64_t i = 0; i < n; ++i) out[i] = x[i] * inv * (double)g[i];
}

/* ------------------------------------------------------------------------ */
/* RoPE ([ENGINE] sections 1 and 4.4; positions per [SWARMKV] section 4)     */
/* v holds n_heads vectors of length hd; each adjacent pair (2i, 2i+1) turns */
/* by pos * theta^(-2i/hd).                                                  */
/* ------------------------------------------------------------------------ */
void orc_rope(double* v, int n_heads, int hd, int64_t pos, double theta) {
    for (int h = 0; h < n_heads; ++h) {
        double* x = v + (int64_t)h * hd;
        for (int i = 0; i < hd / 2; ++i) {
            double freq = pow(theta, -2.0 * (double)i / (double)hd);
            double a = (double)pos * freq;
            double c = cos(a), s = sin(a);
            double x0 = x[2 * i], x1 = x[2 * i + 1];
            x[2 * i] = x0 * c - x1 * s;
            x[2 * i + 1] = x0 * s + x1 * c;
        }
    }
}

double orc_silu(double a) { return a / (1.0 + exp(-a)); }

/* ------------------------------------------------------------------------ */
/* GQA decode attention with causal softmax ([ENGINE] sections 1 and 4.4).   */
/* q [nq][hd] fp64; K, V fp16 laid out [nkv][kv_stride][hd]; keys 0..n_ctx-1 */
/* (n_ctx = pos + 1 for a decode step).  out [nq][hd].                        */
/* ------------------------------------------------------------------------ */
void orc_attention(const double* q, const uint16_t* K, const uint16_t* V, int nq, int nkv, int hd,
                   int64_t kv_stride, int64_t n_ctx, double* out) {
    const int group = nq / nkv;
    const double scale = 1.0 / sqrt((double)hd);
    #pragma omp parallel for schedule(static)
    for (int h = 0; h < nq; ++h) {
        const int g = h / group;
        const uint16_t* Kg = K + (int64_t)g * kv_stride * hd;
        const uint16_t* Vg = V + (int64_t)g * kv_stride * hd;
        const double* qh = q + (int64_t)h * hd;
        double* s = (double*)malloc(sizeof(double) * (size_t)(n_ctx > 0 ? n_ctx : 1));
        double m = -INFINITY;
        for (int64_t t = 0; t < n_ctx; ++t) {
            double dot = 0.0;
            for (int i = 0; i < hd; ++i) dot += qh[i] * orc_f16_to_f64(Kg[t * hd + i]);
            s[t] = dot * scale;
            if (s[t] > m) m = s[t];
        }
        double z = 0.0;
        for (int64_t t = 0; t < n_ctx; ++t) { s[t] = exp(s[t] - m); z += s[t]; }
        double* oh = out + (int64_t)h * hd;
        for (int i = 0; i < hd; ++i) oh[i] = 0.0;
        for (int64_t t = 0; t < n_ctx; ++t) {
            double p = s[t] / z;
            for (int i = 0; i < hd; ++i) oh[i] += p * orc_f16_to_f64(Vg[t * hd + i]);
        }
        free(s);
    }
}

/* Cosine similarity a.b / (|a| |b|) in fp64; 0 when either vector is zero. */
double orc_cosine(const double* a, const double* b, int64_t n) {
    double ab = 0.0, aa = 0.0, bb = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        ab += a[i] * b[i];
        aa += a[i] * a[i];
        bb += b[i] * b[i];
    }
    if (aa == 0.0 || bb == 0.0) return 0.0;
    return ab / (sqrt(aa) * sqrt(bb));
}

/* First index of the largest value after rounding each to fp32 (ties: the
 * lowest index, as the decode step's argmax takes them). */
int32_t orc_argmax_f32(const double* v, int64_t n) {
    int32_t best = 0;
    float bv = (float)v[0];
    for (int64_t i = 1; i < n; ++i) {
        float f = (float)v[i];
        if (f > bv) { bv = f; best = (int32_t)i; }
    }
    return best;
}

/* ------------------------------------------------------------------------ */
/* whole decode step                                                          */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t vocab, hidden, n_layers, n_heads, n_kv_heads, head_dim, ffn;
    double rms_eps, rope_theta;
    int32_t max_ctx, max_seqs, qtype;
} orc_config;

typedef struct {
    const float* attn_norm;
    const float* ffn_norm;
    const uint8_t *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down;
} orc_layer;

typedef struct {
    orc_config c;
    orc_layer* layers;          /* weights are borrowed: the caller keeps them alive */
    const uint16_t* tok_embd;   /* fp16 [vocab][hidden] */
    const float* out_norm;
    const uint8_t* lm_head;
    uint16_t* kcache;           /* [seq][layer][nkv][max_ctx][hd] fp16, owned */
    uint16_t* vcache;
    int64_t* pos;               /* [seq] next position */
} orc_model;

static int64_t kv_index(const orc_model* m, int s, int l) {
    const orc_config* c = &m->c;
    return (((int64_t)s * c->n_layers + l) * c->n_kv_heads) * (int64_t)c->max_ctx * c->head_dim;
}

orc_model* orc_model_create(const orc_config* cfg) {
    orc_model* m = (orc_model*)calloc(1, sizeof(orc_model));
    if (!m) return NULL;
    m->c = *cfg;
    m->layers = (orc_layer*)calloc((size_t)cfg->n_layers, sizeof(orc_layer));
    size_t kv = (size_t)cfg->max_seqs * cfg->n_layers * cfg->n_kv_heads * (size_t)cfg->max_ctx * cfg->head_dim;
    m->kcache = (uint16_t*)calloc(kv ? kv : 1, 2);
    m->vcache = (uint16_t*)calloc(kv ? kv : 1, 2);
    m->pos = (int64_t*)calloc((size_t)cfg->max_seqs, sizeof(int64_t));
    if (!m->layers || !m->kcache || !m->vcache || !m->pos) {
        free(m->layers); free(m->kcache); free(m->vcache); free(m->pos); free(m);
        return NULL;
    }
    return m;
}

void orc_model_destroy(orc_model* m) {
    if (!m) return;
    free(m->layers); free(m->kcache); free(m->vcache); free(m->pos); free(m);
}

void orc_model_set_layer(orc_model* m, int l, const orc_layer* w) { m->layers[l] = *w; }

void orc_model_set_global(orc_model* m, const uint16_t* tok_embd, const float* out_norm, const uint8_t* lm_head) {
    m->tok_embd = tok_embd; m->out_norm = out_norm; m->lm_head = lm_head;
}

/* k, v fp16 [nkv][n_pos][hd]; sets the sequence's next position to n_pos. */
int orc_model_load_kv(orc_model* m, int s, int l, const uint16_t* k, const uint16_t* v, int64_t n_pos) {
    const orc_config* c = &m->c;
    if (s < 0 || s >= c->max_seqs || l < 0 || l >= c->n_layers || n_pos < 0 || n_pos > c->max_ctx) return -1;
    for (int g = 0; g < c->n_kv_heads; ++g)
        for (int64_t t = 0; t < n_pos; ++t)
            for (int i = 0; i < c->head_dim; ++i) {
                int64_t dst = kv_index(m, s, l) + ((int64_t)g * c->max_ctx + t) * c->head_dim + i;
                int64_t src = ((int64_t)g * n_pos + t) * c->head_dim + i;
                m->kcache[dst] = k[src];
                m->vcache[dst] = v[src];
            }
    m->pos[s] = n_pos;
    return 0;
}

/* Copies n_pos cached rows of one (seq, layer) out: fp16 [nkv][n_pos][hd]. */
int orc_model_get_kv(const orc_model* m, int s, int l, uint16_t* k, uint16_t* v, int64_t n_pos) {
    const orc_config* c = &m->c;
    if (s < 0 || s >= c->max_seqs || l < 0 || l >= c->n_layers || n_pos < 0 || n_pos > c->max_ctx) return -1;
    for (int g = 0; g < c->n_kv_heads; ++g)
        for (int64_t t = 0; t < n_pos; ++t)
            for (int i = 0; i < c->head_dim; ++i) {
                int64_t src = kv_index(m, s, l) + ((int64_t)g * c->max_ctx + t) * c->head_dim + i;
                int64_t dst = ((int64_t)g * n_pos + t) * c->head_dim + i;
                k[dst] = m->kcache[src];
                v[dst] = m->vcache[src];
            }
    return 0;
}

int orc_model_set_position(orc_model* m, int s, int64_t pos) {
    if (s < 0 || s >= m->c.max_seqs || pos < 0 || pos > m->c.max_ctx) return -1;
    m->pos[s] = pos;
    return 0;
}

int64_t orc_model_position(const orc_model* m, int s) { return m->pos[s]; }

/*
 * One decode step for n_seq independent sequences (sequence s reads token
 * tokens[s] at position pos[s]).  logits: fp64 [n_seq][vocab] (nullable);
 * argmax: [n_seq].  skip: [n_layers] nonzero = layer skipped (nullable);
 * cos: [n_seq][n_layers] cosine similarity of each computed layer's input and
 * output (nullable; skipped layers get 0).  Returns 0, or -1 on a bad
 * argument / full context.
 */
int orc_decode_step_ex(orc_model* m, const int32_t* tokens, int n_seq, double* logits, int32_t* argmax,
                       const uint8_t* skip, double* cos) {
    const orc_config* c = &m->c;
    const int H = c->hidden, nq = c->n_heads, nkv = c->n_kv_heads, hd = c->head_dim, F = c->ffn;
    if (n_seq < 1 || n_seq > c->max_seqs) return -1;
    for (int s = 0; s < n_seq; ++s) {
        if (tokens[s] < 0 || tokens[s] >= c->vocab) return -1;
        if (m->pos[s] + 1 > c->max_ctx) return -1;
    }
    double* x = (double*)malloc(sizeof(double) * H);
    double* xn = (double*)malloc(sizeof(double) * H);
    double* q = (double*)malloc(sizeof(double) * (size_t)nq * hd);
    double* k = (double*)malloc(sizeof(double) * (size_t)nkv * hd);
    double* v = (double*)malloc(sizeof(double) * (size_t)nkv * hd);
    double* o = (double*)malloc(sizeof(double) * (size_t)nq * hd);
    double* y = (double*)malloc(sizeof(double) * (size_t)(H > F ? H : F));
    double* a = (double*)malloc(sizeof(double) * F);
    double* b = (double*)malloc(sizeof(double) * F);
    double* lg = (double*)malloc(sizeof(double) * c->vocab);
    double* xin = (double*)malloc(sizeof(double) * H);
    int qt = c->qtype;
    for (int s = 0; s < n_seq; ++s) {
        const int64_t p = m->pos[s];
        /* embedding lookup: fp16 row -> fp64 (exact) */
        for (int i = 0; i < H; ++i) x[i] = orc_f16_to_f64(m->tok_embd[(int64_t)tokens[s] * H + i]);
        for (int l = 0; l < c->n_layers; ++l) {
            if (cos) cos[(int64_t)s * c->n_layers + l] = 0.0;
            if (skip && skip[l]) continue;               /* the layer's input is its output */
            memcpy(xin, x, sizeof(double) * H);
            const orc_layer* L = &m->layers[l];
            uint16_t* Kc = m->kcache + kv_index(m, s, l);
            uint16_t* Vc = m->vcache + kv_index(m, s, l);
            /* attention block */
            orc_rmsnorm(x, L->attn_norm, H, c->rms_eps, xn);
            orc_gemv(qt, L->wq, (int64_t)nq * hd, H, xn, q);
            orc_gemv(qt, L->wk, (int64_t)nkv * hd, H, xn, k);
            orc_gemv(qt, L->wv, (int64_t)nkv * hd, H, xn, v);
            orc_rope(q, nq, hd, p, c->rope_theta);
            orc_rope(k, nkv, hd, p, c->rope_theta);
            for (int g = 0; g < nkv; ++g)
                for (int i = 0; i < hd; ++i) {
                    Kc[((int64_t)g * c->max_ctx + p) * hd + i] = orc_f64_to_f16(k[g * hd + i]);
                    Vc[((int64_t)g * c->max_ctx + p) * hd + i] = orc_f64_to_f16(v[g * hd + i]);
                }
            orc_attention(q, Kc, Vc, nq, nkv, hd, c->max_ctx, p + 1, o);
            orc_gemv(qt, L->wo, H, (int64_t)nq * hd, o, y);
            for (int i = 0; i < H; ++i) x[i] += y[i];
            /* feed-forward block: SwiGLU */
            orc_rmsnorm(x, L->ffn_norm, H, c->rms_eps, xn);
            orc_gemv(qt, L->w_gate, F, H, xn, a);
            orc_gemv(qt, L->w_up, F, H, xn, b);
            for (int i = 0; i < F; ++i) a[i] = orc_silu(a[i]) * b[i];
            orc_gemv(qt, L->w_down, H, F, a, y);
            for (int i = 0; i < H; ++i) x[i] += y[i];
            if (cos) cos[(int64_t)s * c->n_layers + l] = orc_cosine(xin, x, H);
        }
        orc_rmsnorm(x, m->out_norm, H, c->rms_eps, xn);
        orc_gemv(qt, m->lm_head, c->vocab, H, xn, lg);
        if (logits) memcpy(logits + (int64_t)s * c->vocab, lg, sizeof(double) * c->vocab);
        argmax[s] = orc_argmax_f32(lg, c->vocab);
        m->pos[s] = p + 1;
    }
    free(x); free(xn); free(q); free(k); free(v); free(o); free(y); free(a); free(b); free(lg); free(xin);
    return 0;
}

int orc_decode_step(orc_model* m, const int32_t* tokens, int n_seq, double* logits, int32_t* argmax) {
    return orc_decode_step_ex(m, tokens, n_seq, logits, argmax, NULL, NULL);
}

/*
 * Self-speculative acceptance ([ENGINE] sections 3.5 and 5.3: draft tokens
 * with the bottom layers, then verify them with the full model).  draft[0..k-1]
 * are the drafted tokens d1..dk; verify[0..k] the full model's argmax after
 * [t0, d1, .., dk] at positions p..p+k.  The longest prefix d1..di with
 * verify[j] == d(j+1) for every j < i is accepted, then verify[i] (the full
 * model's own next token) is appended: out[0..i], returns i + 1.  Greedy
 * decoding gives the same tokens.
 */
int orc_spec_accept(const int32_t* draft, const int32_t* verify, int k, int32_t* out) {
    int i = 0;
    while (i < k && verify[i] == draft[i]) {
        out[i] = draft[i];
        ++i;
    }
    out[i] = verify[i];
    return i + 1;
}

/* The calibrated skip list: mask[l] = 1 when mean_cos[l] > threshold. */
int orc_skip_list(const double* mean_cos, int n_layers, double threshold, uint8_t* mask) {
    int n = 0;
    for (int l = 0; l < n_layers; ++l) {
        mask[l] = mean_cos[l] > threshold;
        n += mask[l];
    }
    return n;
}
