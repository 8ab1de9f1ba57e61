/*
 * synth.c - seeded synthetic inputs for the quantized Llama decode step.
 *
 * This module only MAKES inputs: random numbers, random models already cast
 * into the GGUF Q8_0 / Q4_0 block formats, fp16 tables, token ids.  It holds
 * none of the decode step's arithmetic (no dequantisation, no matvec, no
 * normalisation, no attention).  Both the fp64 oracle and the HIP library
 * consume the bytes written here, and neither side links this file.
 *
 * Random numbers: Philox4x32-10, the counter-based generator published by
 * Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3"
 * (SC'11).  Key = (seed, tensor id), counter = element index / 4, so every
 * element has a fixed value whatever the thread count or the chunking.
 * Normals come from the Box-Muller transform of two uniforms in (0, 1).
 *
 * Block formats (page "rskf.cn/news/15116", section 1 names Q8_0 and Q4_0
 * among the GGUF formats the engine reads; the recipe below is the one the
 * workload definition states):
 *   Q8_0: 32 weights along the input dimension; fp16 d = max|w|/127 stored
 *         first, then 32 int8 q = round(w/d).  34 bytes per block.
 *   Q4_0: 32 weights; fp16 d = max|w|/7, then 16 bytes; q = clamp(round(w/d)
 *         + 8, 0, 15); byte j holds element j in its low nibble and element
 *         j+16 in its high nibble.  18 bytes per block.
 * round() is half away from zero (C roundf); q uses the fp32 d before it is
 * rounded to fp16; an all-zero block has d = 0 and q = 0 (Q8_0) / 8 (Q4_0).
 *
 * The GGUF "K" formats (the same page names Q4_K and Q6_K, the formats of its
 * 70B figures, without defining them; the byte layout is GGUF's published
 * one): 256-weight super-blocks.  This generator's own recipe:
 *   Q4_K (144 bytes): per 32-weight sub-block j, mn_j = max(0, -min w) and
 *         s_j = (max w + mn_j)/15; d = max_j s_j / 63, dmin = max_j mn_j / 63
 *         (fp32, stored fp16); sc_j = round(s_j/d), m_j = round(mn_j/dmin)
 *         clamped to 0..63; q = clamp(round((w + dmin*m_j)/(d*sc_j)), 0, 15).
 *         Layout: fp16 d, fp16 dmin, 12 bytes of packed 6-bit sc/m, 128 bytes
 *         of nibbles (bytes 32g..32g+31 hold sub-block 2g in their low
 *         nibbles and sub-block 2g+1 in their high nibbles).
 *   Q5_K (176 bytes): as Q4_K with 31 steps per sub-block instead of 15
 *         (q = clamp(round((w + dmin*m_j)/(d*sc_j)), 0, 31)).  Layout: the
 *         Q4_K header, 32 bytes of fifth bits (bit j of byte l: element
 *         32j + l), 128 bytes of low nibbles grouped as in Q4_K.
 *   Q6_K (210 bytes): per 16-weight sub-block k, s_k = max|w|/31;
 *         d = max_k s_k / 127; sc_k = round(s_k/d) (0..127, stored int8);
 *         q = clamp(round(w/(d*sc_k)), -32, 31) + 32.  Layout: 128 bytes of
 *         low nibbles, 64 bytes of 2-bit high parts, 16 int8 scales, fp16 d.
 * d, dmin and the sub-block scales use the fp32 values before any rounding;
 * a zero scale gives q = 0 (Q4_K) / 32 (Q6_K).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYN_Q4_0 2
#define SYN_Q8_0 8
#define SYN_Q4_K 12
#define SYN_Q5_K 13
#define SYN_Q6_K 14

/* ---- Philox4x32-10 (Salmon et al. SC'11, section 3.2 / table 2 constants) */
static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

void synth_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo32(M0, c0, &hi0, &lo0);
        mulhilo32(M1, c2, &hi1, &lo1);
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += W0; k1 += W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline void stream_key(uint64_t seed, uint64_t tensor_id, uint32_t key[2]) {
    /* 32 bits of seed and 32 bits of tensor id; both are small in practice. */
    key[0] = (uint32_t)(seed ^ (seed >> 32));
    key[1] = (uint32_t)(tensor_id ^ (tensor_id >> 32));
}

static inline void block4(const uint32_t key[2], uint64_t c, uint32_t out[4]) {
    uint32_t ctr[4] = {(uint32_t)c, (uint32_t)(c >> 32), 0u, 0u};
    synth_philox4x32_10(ctr, key, out);
}

/* Four standard normals from counter c (two Box-Muller pairs). */
static inline void normals4(const uint32_t key[2], uint64_t c, double z[4]) {
    uint32_t u[4];
    block4(key, c, u);
    const double s = 2.3283064365386963e-10; /* 2^-32 */
    const double two_pi = 6.283185307179586476925286766559;
    for (int p = 0; p < 2; ++p) {
        double u1 = ((double)u[2 * p] + 0.5) * s;     /* (0, 1) */
        double u2 = ((double)u[2 * p + 1] + 0.5) * s;
        double r = sqrt(-2.0 * log(u1));
        z[2 * p] = r * cos(two_pi * u2);
        z[2 * p + 1] = r * sin(two_pi * u2);
    }
}

/* Element i of the standard-normal stream (seed, tensor_id). */
static inline double normal_at(const uint32_t key[2], uint64_t i, uint64_t* cached_c, double cache[4]) {
    uint64_t c = i >> 2;
    if (c != *cached_c) {
        normals4(key, c, cache);
        *cached_c = c;
    }
    return cache[i & 3];
}

/* ---- fp16 (IEEE binary16) encoding, round to nearest even ---------------- */
uint16_t synth_f64_to_f16(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7E00u);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00u); /* rounds to inf */
    if (a < 6.103515625e-05) {                            /* below 2^-14: subnormal */
        double m = a * 16777216.0;                        /* units of 2^-24 */
        double r = nearbyint(m);                          /* default mode: ties to even */
        return (uint16_t)(sign | (uint16_t)r);            /* r == 1024 encodes 2^-14 */
    }
    int e;
    double f = frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) */
    double m = f * 2048.0;            /* 11 significant bits incl. the leading one */
    double r = nearbyint(m);
    if (r == 2048.0) { r = 1024.0; e += 1; }
    int exp16 = e - 1 + 15;
    if (exp16 >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | (uint16_t)(exp16 << 10) | ((uint16_t)r & 0x3FFu));
}

/* ---- block quantisers ---------------------------------------------------- */
static void quant_block_q8_0(const float* w, uint8_t* out) {
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) { float a = fabsf(w[j]); if (a > amax) amax = a; }
    float d = amax / 127.0f;
    uint16_t dh = synth_f64_to_f16((double)d);
    memcpy(out, &dh, 2);
    int8_t* q = (int8_t*)(out + 2);
    for (int j = 0; j < 32; ++j) {
        int v = 0;
        if (d != 0.0f) {
            v = (int)roundf(w[j] / d);
            if (v > 127) v = 127;
            if (v < -127) v = -127;
        }
        q[j] = (int8_t)v;
    }
}

static void quant_block_q4_0(const float* w, uint8_t* out) {
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) { float a = fabsf(w[j]); if (a > amax) amax = a; }
    float d = amax / 7.0f;
    uint16_t dh = synth_f64_to_f16((double)d);
    memcpy(out, &dh, 2);
    int q[32];
    for (int j = 0; j < 32; ++j) {
        int v = 8;
        if (d != 0.0f) {
            v = (int)roundf(w[j] / d) + 8;
            if (v > 15) v = 15;
            if (v < 0) v = 0;
        }
        q[j] = v;
    }
    for (int j = 0; j < 16; ++j) out[2 + j] = (uint8_t)(q[j] | (q[j + 16] << 4));
}

/* Q4_K (levels 15) and Q5_K (levels 31): shared header recipe */
static void quant_block_kmin(const float* w, uint8_t* out, int levels);
static void quant_block_q4_k(const float* w, uint8_t* out) { quant_block_kmin(w, out, 15); }
static void quant_block_q5_k(const float* w, uint8_t* out) { quant_block_kmin(w, out, 31); }

static void quant_block_kmin(const float* w, uint8_t* out, int levels) {
    float s[8], mn[8], smax = 0.0f, mmax = 0.0f;
    for (int j = 0; j < 8; ++j) {
        float lo = w[32 * j], hi = w[32 * j];
        for (int i = 1; i < 32; ++i) {
            if (w[32 * j + i] < lo) lo = w[32 * j + i];
            if (w[32 * j + i] > hi) hi = w[32 * j + i];
        }
        mn[j] = lo < 0.0f ? -lo : 0.0f;
        s[j] = (hi + mn[j]) / (float)levels;
        if (s[j] > smax) smax = s[j];
        if (mn[j] > mmax) mmax = mn[j];
    }
    const float d = smax / 63.0f, dmin = mmax / 63.0f;
    uint16_t dh = synth_f64_to_f16((double)d), mh = synth_f64_to_f16((double)dmin);
    memcpy(out, &dh, 2);
    memcpy(out + 2, &mh, 2);
    int sc[8], m[8];
    for (int j = 0; j < 8; ++j) {
        int a = d > 0.0f ? (int)roundf(s[j] / d) : 0, b = dmin > 0.0f ? (int)roundf(mn[j] / dmin) : 0;
        sc[j] = a < 0 ? 0 : (a > 63 ? 63 : a);
        m[j] = b < 0 ? 0 : (b > 63 ? 63 : b);
    }
    uint8_t* p = out + 4;
    for (int j = 0; j < 4; ++j) {
        p[j] = (uint8_t)(sc[j] | ((sc[j + 4] >> 4) << 6));
        p[j + 4] = (uint8_t)(m[j] | ((m[j + 4] >> 4) << 6));
        p[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
    }
    int q[256];
    for (int e = 0; e < 256; ++e) {
        const int j = e / 32;
        const float es = d * (float)sc[j], em = dmin * (float)m[j];
        int v = 0;
        if (es > 0.0f) {
            v = (int)roundf((w[e] + em) / es);
            if (v < 0) v = 0;
            if (v > levels) v = levels;
        }
        q[e] = v;
    }
    uint8_t* qs = out + (levels == 15 ? 16 : 48);
    for (int g = 0; g < 4; ++g)
        for (int l = 0; l < 32; ++l)
            qs[32 * g + l] = (uint8_t)((q[64 * g + l] & 15) | ((q[64 * g + 32 + l] & 15) << 4));
    if (levels == 31) {
        uint8_t* qh = out + 16;
        memset(qh, 0, 32);
        for (int e = 0; e < 256; ++e) qh[e % 32] |= (uint8_t)(((q[e] >> 4) & 1) << (e / 32));
    }
}

static void quant_block_q6_k(const float* w, uint8_t* out) {
    float s[16], smax = 0.0f;
    for (int k = 0; k < 16; ++k) {
        float amax = 0.0f;
        for (int i = 0; i < 16; ++i) { float a = fabsf(w[16 * k + i]); if (a > amax) amax = a; }
        s[k] = amax / 31.0f;
        if (s[k] > smax) smax = s[k];
    }
    const float d = smax / 127.0f;
    int sc[16];
    for (int k = 0; k < 16; ++k) {
        int a = d > 0.0f ? (int)roundf(s[k] / d) : 0;
        sc[k] = a < 0 ? 0 : (a > 127 ? 127 : a);
    }
    uint8_t* ql = out;
    uint8_t* qh = out + 128;
    memset(out, 0, 192);
    for (int e = 0; e < 256; ++e) {
        const float es = d * (float)sc[e / 16];
        int v = 32;
        if (es > 0.0f) {
            v = (int)roundf(w[e] / es);
            if (v < -32) v = -32;
            if (v > 31) v = 31;
            v += 32;
        }
        const int h = e / 128, r = e % 128, t = r / 32, l = r % 32;
        ql[64 * h + l + 32 * (t % 2)] |= (uint8_t)((v & 15) << (t < 2 ? 0 : 4));
        qh[32 * h + l] |= (uint8_t)((v >> 4) << (2 * t));
    }
    for (int k = 0; k < 16; ++k) out[192 + k] = (uint8_t)(int8_t)sc[k];
    uint16_t dh = synth_f64_to_f16((double)d);
    memcpy(out + 208, &dh, 2);
}

static int block_bytes(int qtype) {
    switch (qtype) {
        case SYN_Q8_0: return 34;
        case SYN_Q4_0: return 18;
        case SYN_Q4_K: return 144;
        case SYN_Q5_K: return 176;
        case SYN_Q6_K: return 210;
        default: return -1;
    }
}
static int block_weights(int qtype) {
    return qtype == SYN_Q4_K || qtype == SYN_Q5_K || qtype == SYN_Q6_K ? 256 : 32;
}

static void quant_block(int qtype, const float* w, uint8_t* out) {
    switch (qtype) {
        case SYN_Q8_0: quant_block_q8_0(w, out); break;
        case SYN_Q4_0: quant_block_q4_0(w, out); break;
        case SYN_Q4_K: quant_block_q4_k(w, out); break;
        case SYN_Q5_K: quant_block_q5_k(w, out); break;
        default: quant_block_q6_k(w, out); break;
    }
}

/* Quantise n fp32 values (n a multiple of the block size) into consecutive blocks. */
int synth_quantize(const float* w, int64_t n, int qtype, uint8_t* out) {
    const int bb = block_bytes(qtype), qk = block_weights(qtype);
    if (bb < 0 || n % qk != 0) return -1;
    for (int64_t b = 0; b < n / qk; ++b) quant_block(qtype, w + qk * b, out + bb * b);
    return 0;
}

/* ---- random tensors ------------------------------------------------------ */
/* out[i] = (float)(mean + std * z_{offset+i}) */
void synth_normal_f32(uint64_t seed, uint64_t tensor_id, int64_t offset, int64_t n,
                      double mean, double std, float* out) {
    uint32_t key[2];
    stream_key(seed, tensor_id, key);
    #pragma omp parallel
    {
        uint64_t cc = UINT64_MAX;
        double cache[4];
        #pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i)
            out[i] = (float)(mean + std * normal_at(key, (uint64_t)(offset + i), &cc, cache));
    }
}

/* out[i] = fp16_rne(mean + std * z_{offset+i}) as raw bits */
void synth_normal_f16(uint64_t seed, uint64_t tensor_id, int64_t offset, int64_t n,
                      double mean, double std, uint16_t* out) {
    uint32_t key[2];
    stream_key(seed, tensor_id, key);
    #pragma omp parallel
    {
        uint64_t cc = UINT64_MAX;
        double cache[4];
        #pragma omp for schedule(static)
        for (int64_t i = 0; i < n; ++i)
            out[i] = synth_f64_to_f16(mean + std * normal_at(key, (uint64_t)(offset + i), &cc, cache));
    }
}

/* Uniform integers in [0, bound): raw Philox word modulo bound. */
void synth_uniform_int(uint64_t seed, uint64_t tensor_id, int64_t n, uint32_t bound, int32_t* out) {
    uint32_t key[2];
    stream_key(seed, tensor_id, key);
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u[4];
        block4(key, (uint64_t)i >> 2, u);
        out[i] = (int32_t)(u[i & 3] % bound);
    }
}

/*
 * A rows x cols weight matrix with entries (float)(std * z), quantised block by
 * block as it is drawn (row-major, blocks of 32 along cols).  Element (r, c) is
 * element r*cols + c of the stream, so a block never depends on the chunking.
 */
int synth_quant_matrix(uint64_t seed, uint64_t tensor_id, int64_t rows, int64_t cols,
                       double std, int qtype, uint8_t* out) {
    const int bb = block_bytes(qtype), qk = block_weights(qtype);
    if (bb < 0 || cols % qk != 0 || rows < 0) return -1;
    uint32_t key[2];
    stream_key(seed, tensor_id, key);
    const int64_t nb = cols / qk;
    const int64_t total = rows * nb;
    #pragma omp parallel
    {
        float w[256];
        #pragma omp for schedule(static)
        for (int64_t blk = 0; blk < total; ++blk) {
            uint64_t base = (uint64_t)blk * (uint64_t)qk; /* = r*cols + b*qk */
            /* qk consecutive elements = qk/4 Philox counters, aligned to 4 */
            for (int c4 = 0; c4 < qk / 4; ++c4) {
                double z[4];
                normals4(key, (base >> 2) + (uint64_t)c4, z);
                for (int t = 0; t < 4; ++t) w[4 * c4 + t] = (float)(std * z[t]);
            }
            quant_block(qtype, w, out + bb * blk);
        }
    }
    return 0;
}
