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
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYN_Q4_0 2
#define SYN_Q8_0 8

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

static int block_bytes(int qtype) {
    return qtype == SYN_Q8_0 ? 34 : (qtype == SYN_Q4_0 ? 18 : -1);
}

/* Quantise n fp32 values (n a multiple of 32) into consecutive blocks. */
int synth_quantize(const float* w, int64_t n, int qtype, uint8_t* out) {
    int bb = block_bytes(qtype);
    if (bb < 0 || n % 32 != 0) return -1;
    for (int64_t b = 0; b < n / 32; ++b) {
        if (qtype == SYN_Q8_0) quant_block_q8_0(w + 32 * b, out + bb * b);
        else quant_block_q4_0(w + 32 * b, out + bb * b);
    }
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
    int bb = block_bytes(qtype);
    if (bb < 0 || cols % 32 != 0 || rows < 0) return -1;
    uint32_t key[2];
    stream_key(seed, tensor_id, key);
    const int64_t nb = cols / 32;
    const int64_t total = rows * nb;
    #pragma omp parallel
    {
        float w[32];
        #pragma omp for schedule(static)
        for (int64_t blk = 0; blk < total; ++blk) {
            uint64_t base = (uint64_t)blk * 32u; /* = r*cols + b*32 */
            /* 32 consecutive elements = 8 Philox counters, aligned to 4 */
            for (int c4 = 0; c4 < 8; ++c4) {
                double z[4];
                normals4(key, (base >> 2) + (uint64_t)c4, z);
                for (int t = 0; t < 4; ++t) w[4 * c4 + t] = (float)(std * z[t]);
            }
            if (qtype == SYN_Q8_0) quant_block_q8_0(w, out + bb * blk);
            else quant_block_q4_0(w, out + bb * blk);
        }
    }
    return 0;
}
