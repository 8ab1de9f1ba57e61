// lm_kernels.hip - gfx950 kernels of the batch-1 quantised Llama decode step.
//
// Operators (C/CUDA Llama engine page, rskf.cn/news/15116, section 4.4):
// a GEMV specialised for the single-token vector x matrix product, RMSNorm
// fused with its gain, RoPE from a precomputed sin/cos table fused into the
// producing operator, SwiGLU fused with the fully connected product, and a
// softmax with the causal mask folded in.  Block formats Q8_0 / Q4_0 and the
// Llama features (GQA, KV cache) are listed in section 1 of the same page.
//
// MI355X design (CDNA4, 64-lane wavefronts, 160 KB LDS per CU):
//  * dequant-GEMV: a wavefront owns two adjacent output rows at a time
//    (so a RoPE pair or a gate/up pair ends in the same lanes); 64/LPR row
//    pairs share a wavefront when K is short.  Quants arrive as coalesced
//    16-byte loads from the repacked half-block planes; the activation vector
//    sits in LDS in fp32, XOR-swizzled per 32-column block so lanes reading
//    consecutive blocks hit distinct banks.  fp32 accumulation; int8 -> fp32
//    through the SDWA sign-extending convert; partial sums reduced across
//    lanes with cross-lane shuffles.  The RMSNorm of the input is computed
//    by every workgroup while it stages x (prologue); RoPE + fp16 KV append,
//    SwiGLU, residual add, or logits + argmax run in the epilogue.
//  * attention: one workgroup per (64-position chunk, KV head, sequence)
//    stages its K/V tile in LDS once for all query heads of the group; the
//    last workgroup of a (sequence, KV head) to finish merges the chunks'
//    partial softmax states (log-sum-exp) - no second launch.
#include "lm_internal.h"

#include <float.h>
#include <limits.h>

#include <algorithm>

namespace lmk {

constexpr int kBlock = 256;   // threads per workgroup (4 wavefronts)
constexpr int kWaves = kBlock / 64;

// ---------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xswz(int i) {
    // column i -> LDS slot: block b = i/32 keeps its 32 floats, its eight
    // 16-byte chunks are permuted by XOR with (b & 7)
    const int b = i >> 5, j = (i >> 2) & 7;
    return (b << 5) | ((j ^ (b & 7)) << 2) | (i & 3);
}

__device__ __forceinline__ float i8f(uint32_t v, int k) { return (float)(int8_t)(v >> (8 * k)); }
__device__ __forceinline__ float u8f(uint32_t v, int k) { return (float)((v >> (8 * k)) & 0xFFu); }

// 16-byte streaming load (weights are read once per token: non-temporal hint)
typedef int v4i_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int4 ld16_stream(const uint8_t* p) {
#if LMK_WEIGHT_NT
    const v4i_t v = __builtin_nontemporal_load((const v4i_t*)p);
#else
    const v4i_t v = *(const v4i_t*)p;
#endif
    return make_int4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float h2f(uint16_t h) {
    return __half2float(__ushort_as_half(h));
}

__device__ __forceinline__ float wave_sum(float v) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// (value, index) maximum with the lowest index winning ties
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
    if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

__device__ __forceinline__ float dot4(float4 x, float a, float b, float c, float d, float acc) {
    acc = fmaf(a, x.x, acc);
    acc = fmaf(b, x.y, acc);
    acc = fmaf(c, x.z, acc);
    acc = fmaf(d, x.w, acc);
    return acc;
}

// 32 int8 weights (two 16-byte halves) against the block's 32 activations
__device__ __forceinline__ float dot_q8(const int4 A, const int4 B, const float* xb, int sw) {
    const float4 x0 = *(const float4*)(xb + ((0 ^ sw) << 2));
    const float4 x1 = *(const float4*)(xb + ((1 ^ sw) << 2));
    const float4 x2 = *(const float4*)(xb + ((2 ^ sw) << 2));
    const float4 x3 = *(const float4*)(xb + ((3 ^ sw) << 2));
    const float4 x4 = *(const float4*)(xb + ((4 ^ sw) << 2));
    const float4 x5 = *(const float4*)(xb + ((5 ^ sw) << 2));
    const float4 x6 = *(const float4*)(xb + ((6 ^ sw) << 2));
    const float4 x7 = *(const float4*)(xb + ((7 ^ sw) << 2));
    const uint32_t a0 = A.x, a1 = A.y, a2 = A.z, a3 = A.w;
    const uint32_t b0 = B.x, b1 = B.y, b2 = B.z, b3 = B.w;
    float t0 = dot4(x0, i8f(a0, 0), i8f(a0, 1), i8f(a0, 2), i8f(a0, 3), 0.f);
    float t1 = dot4(x1, i8f(a1, 0), i8f(a1, 1), i8f(a1, 2), i8f(a1, 3), 0.f);
    float t2 = dot4(x2, i8f(a2, 0), i8f(a2, 1), i8f(a2, 2), i8f(a2, 3), 0.f);
    float t3 = dot4(x3, i8f(a3, 0), i8f(a3, 1), i8f(a3, 2), i8f(a3, 3), 0.f);
    t0 = dot4(x4, i8f(b0, 0), i8f(b0, 1), i8f(b0, 2), i8f(b0, 3), t0);
    t1 = dot4(x5, i8f(b1, 0), i8f(b1, 1), i8f(b1, 2), i8f(b1, 3), t1);
    t2 = dot4(x6, i8f(b2, 0), i8f(b2, 1), i8f(b2, 2), i8f(b2, 3), t2);
    t3 = dot4(x7, i8f(b3, 0), i8f(b3, 1), i8f(b3, 2), i8f(b3, 3), t3);
    return (t0 + t1) + (t2 + t3);
}

// 32 4-bit weights (16 bytes, GGUF nibble order) against the block's
// activations; returns sum(n_j * x_j), the caller subtracts 8 * sum(x)
__device__ __forceinline__ float dot_q4(const int4 A, const float* xb, int sw) {
    const float4 x0 = *(const float4*)(xb + ((0 ^ sw) << 2));
    const float4 x1 = *(const float4*)(xb + ((1 ^ sw) << 2));
    const float4 x2 = *(const float4*)(xb + ((2 ^ sw) << 2));
    const float4 x3 = *(const float4*)(xb + ((3 ^ sw) << 2));
    const float4 x4 = *(const float4*)(xb + ((4 ^ sw) << 2));
    const float4 x5 = *(const float4*)(xb + ((5 ^ sw) << 2));
    const float4 x6 = *(const float4*)(xb + ((6 ^ sw) << 2));
    const float4 x7 = *(const float4*)(xb + ((7 ^ sw) << 2));
    const uint32_t w0 = A.x, w1 = A.y, w2 = A.z, w3 = A.w;
    const uint32_t l0 = w0 & 0x0F0F0F0Fu, h0 = (w0 >> 4) & 0x0F0F0F0Fu;
    const uint32_t l1 = w1 & 0x0F0F0F0Fu, h1 = (w1 >> 4) & 0x0F0F0F0Fu;
    const uint32_t l2 = w2 & 0x0F0F0F0Fu, h2 = (w2 >> 4) & 0x0F0F0F0Fu;
    const uint32_t l3 = w3 & 0x0F0F0F0Fu, h3 = (w3 >> 4) & 0x0F0F0F0Fu;
    float t0 = dot4(x0, u8f(l0, 0), u8f(l0, 1), u8f(l0, 2), u8f(l0, 3), 0.f);
    float t1 = dot4(x1, u8f(l1, 0), u8f(l1, 1), u8f(l1, 2), u8f(l1, 3), 0.f);
    float t2 = dot4(x2, u8f(l2, 0), u8f(l2, 1), u8f(l2, 2), u8f(l2, 3), 0.f);
    float t3 = dot4(x3, u8f(l3, 0), u8f(l3, 1), u8f(l3, 2), u8f(l3, 3), 0.f);
    t0 = dot4(x4, u8f(h0, 0), u8f(h0, 1), u8f(h0, 2), u8f(h0, 3), t0);
    t1 = dot4(x5, u8f(h1, 0), u8f(h1, 1), u8f(h1, 2), u8f(h1, 3), t1);
    t2 = dot4(x6, u8f(h2, 0), u8f(h2, 1), u8f(h2, 2), u8f(h2, 3), t2);
    t3 = dot4(x7, u8f(h3, 0), u8f(h3, 1), u8f(h3, 2), u8f(h3, 3), t3);
    return (t0 + t1) + (t2 + t3);
}

__device__ __forceinline__ float block_sum(float v, float* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = 0.f;
    #pragma unroll
    for (int w = 0; w < kWaves; ++w) t += red[w];
    return t;
}

// ---------------------------------------------------------------------------
// embedding: x[s] = fp32(E[token[s]])
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_embed(const uint16_t* __restrict__ E,
                                                 const int* __restrict__ tokens, int vocab,
                                                 int hidden, float* __restrict__ x) {
    const int s = blockIdx.y;
    int t = tokens[s];
    if (t < 0 || t >= vocab) t = 0;
    const int i = (blockIdx.x * kBlock + threadIdx.x) * 4;
    if (i >= hidden) return;
    const uint2 raw = *(const uint2*)(E + (int64_t)t * hidden + i);
    float4 v;
    v.x = h2f((uint16_t)(raw.x & 0xFFFF));
    v.y = h2f((uint16_t)(raw.x >> 16));
    v.z = h2f((uint16_t)(raw.y & 0xFFFF));
    v.w = h2f((uint16_t)(raw.y >> 16));
    *(float4*)(x + (int64_t)s * hidden + i) = v;
}

hipError_t launch_embed(const uint16_t* tok_embd, const int* tokens, int vocab, int hidden,
                        float* x, int n_seq, hipStream_t st) {
    dim3 grid((hidden / 4 + kBlock - 1) / kBlock, n_seq);
    hipLaunchKernelGGL(k_embed, grid, dim3(kBlock), 0, st, tok_embd, tokens, vocab, hidden, x);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dequant-GEMV with fused prologue / epilogue
// ---------------------------------------------------------------------------
// Tuning knobs (compile-time): blocks per lane per pipeline stage, and
// whether weight loads carry the non-temporal hint.
#ifndef LMK_CB_Q8
#define LMK_CB_Q8 2
#endif
#ifndef LMK_CB_Q4
#define LMK_CB_Q4 4
#endif
#ifndef LMK_WEIGHT_NT
#define LMK_WEIGHT_NT 1
#endif

// Weight blocks one lane loads per pipeline stage (per row of its row pair).
template <int QT> struct ChunkBlocks { static constexpr int value = LMK_CB_Q8; };
template <> struct ChunkBlocks<kQ4_0> { static constexpr int value = LMK_CB_Q4; };

// One pipeline stage of a lane: CB blocks of both rows of its row pair.
template <int QT>
struct WChunk {
    static constexpr int CB = ChunkBlocks<QT>::value;
    int4 a0[CB], a1[CB];          // first 16 bytes (Q8_0) / all 16 bytes (Q4_0) of row 0 / row 1
    int4 b0[QT == kQ8_0 ? CB : 1], b1[QT == kQ8_0 ? CB : 1];   // Q8_0 second halves
    uint16_t d0[CB], d1[CB];
};

#ifndef LMK_GEMV_MIN_BLOCKS
#define LMK_GEMV_MIN_BLOCKS 1     // workgroups per CU the register budget must allow
#endif

template <int QT, int LPR, int EPI>
__global__ __launch_bounds__(kBlock, LMK_GEMV_MIN_BLOCKS) void k_gemv(GemvArgs a) {
    extern __shared__ __align__(16) float smem[];
    __shared__ float red[kWaves];
    __shared__ float wv_best[kWaves];
    __shared__ int wi_best[kWaves];
    __shared__ int s_last;

    constexpr int CB = ChunkBlocks<QT>::value;
    constexpr int kGroups = 64 / LPR;            // row pairs per wavefront step
    constexpr int kRowsPerStep = 2 * kGroups;

    const int K = a.w.K, N = a.w.N, nb = K >> 5;
    float* xs = smem;            // K floats, swizzled
    float* bsum = smem + K;      // nb block sums (Q4_0)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int s = blockIdx.y;
    const float* x = a.xin + (int64_t)s * a.x_stride;
    const int rg = lane / LPR, li = lane % LPR;
    const int64_t rowq = (QT == kQ8_0) ? (int64_t)K : (int64_t)(K >> 1);

    // this wavefront's steps: step0, step0 + sstride, ... ; each step is split
    // into `cps` chunks of CB blocks per lane
    const int n_steps = (N + kRowsPerStep - 1) / kRowsPerStep;
    const int step0 = blockIdx.x * kWaves + wave, sstride = gridDim.x * kWaves;
    const int my_steps = step0 < n_steps ? (n_steps - 1 - step0) / sstride + 1 : 0;
    const int bpl = (nb + LPR - 1) / LPR;        // blocks per lane per row (upper bound)
    const int cps = (bpl + CB - 1) / CB;
    const int n_chunks = my_steps * cps;

    // ---- RoPE inputs of this wavefront's first row pair, fetched early
    int rope_p = 0;
    float pre_cs = 1.f, pre_sn = 0.f;
    if (EPI == EPI_QKV) {
        rope_p = a.pos[s];
        const int r0 = step0 * kRowsPerStep + rg * 2;
        if (n_chunks > 0 && li == 0 && r0 < a.q_rows + a.kv_rows) {
            const int rr = r0 < a.q_rows ? r0 : r0 - a.q_rows;
            const int pi = (rr % a.head_dim) >> 1;
            pre_cs = a.rope_cos[(int64_t)rope_p * (a.head_dim >> 1) + pi];
            pre_sn = a.rope_sin[(int64_t)rope_p * (a.head_dim >> 1) + pi];
        }
    }

    // Branch-free loads (clamped addresses; a block past the row end gets
    // scale 0) so the compiler's in-order load counters stay exact and the
    // next chunk's loads remain in flight while this one computes.
    auto load = [&](int c, WChunk<QT>& w) {
        const int i = c / cps, k = c - i * cps;
        const int r0 = min((step0 + i * sstride) * kRowsPerStep + rg * 2, N - 2);
        const uint8_t* q0 = a.w.q + (int64_t)r0 * rowq;
        const uint8_t* q1 = q0 + rowq;
        const uint16_t* s0 = a.w.sc + (int64_t)r0 * nb;
        #pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int b = li + LPR * (k * CB + u);
            const int bc = min(b, nb - 1);
            w.a0[u] = ld16_stream(q0 + bc * 16);
            w.a1[u] = ld16_stream(q1 + bc * 16);
            if (QT == kQ8_0) {
                w.b0[u] = ld16_stream(q0 + (int64_t)nb * 16 + bc * 16);
                w.b1[u] = ld16_stream(q1 + (int64_t)nb * 16 + bc * 16);
            }
            w.d0[u] = s0[bc];          // used only in compute(): consuming a load here
            w.d1[u] = s0[nb + bc];     // would wait on every load issued before it
        }
    };

    float acc0 = 0.f, acc1 = 0.f;
    auto compute = [&](int c, const WChunk<QT>& w) {
        const int k = c % cps;
        #pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int braw = li + LPR * (k * CB + u);
            const int b = min(braw, nb - 1);
            const float d0 = braw < nb ? h2f(w.d0[u]) : 0.f;   // past the row end: no contribution
            const float d1 = braw < nb ? h2f(w.d1[u]) : 0.f;
            const float* xb = xs + (b << 5);
            const int sw = b & 7;
            if (QT == kQ8_0) {
                acc0 = fmaf(d0, dot_q8(w.a0[u], w.b0[u], xb, sw), acc0);
                acc1 = fmaf(d1, dot_q8(w.a1[u], w.b1[u], xb, sw), acc1);
            } else {
                const float c8 = 8.f * bsum[b];
                acc0 = fmaf(d0, dot_q4(w.a0[u], xb, sw) - c8, acc0);
                acc1 = fmaf(d1, dot_q4(w.a1[u], xb, sw) - c8, acc1);
            }
        }
    };

    float best_v = -FLT_MAX;
    int best_i = INT_MAX;
    float rscale = 1.f;   // RMSNorm factor of the input (1 without a gain)

    // after the last chunk of a step: reduce the row pair across its lanes, then the epilogue
    auto finish = [&](int c) {
        if (c % cps != cps - 1) return;
        const int i = c / cps;
        const int r0 = (step0 + i * sstride) * kRowsPerStep + rg * 2;
        #pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) {
            acc0 += __shfl_xor(acc0, off, 64);
            acc1 += __shfl_xor(acc1, off, 64);
        }
        const float y0 = acc0 * rscale, y1 = acc1 * rscale;
        acc0 = 0.f;
        acc1 = 0.f;
        if (li != 0 || r0 >= N) return;
        if (EPI == EPI_QKV) {
            const int p = rope_p;
            const int hd = a.head_dim;
            if (r0 < a.q_rows + a.kv_rows) {
                // RoPE on (2i, 2i+1) of the head, angle p * theta^(-2i/hd)
                const int rr = r0 < a.q_rows ? r0 : r0 - a.q_rows;
                const int pi = (rr % hd) >> 1;
                const float cs = i == 0 ? pre_cs : a.rope_cos[(int64_t)p * (hd >> 1) + pi];
                const float sn = i == 0 ? pre_sn : a.rope_sin[(int64_t)p * (hd >> 1) + pi];
                const float z0 = y0 * cs - y1 * sn;
                const float z1 = y0 * sn + y1 * cs;
                if (r0 < a.q_rows) {
                    *(float2*)(a.out + (int64_t)s * a.out_stride + r0) = make_float2(z0, z1);
                } else {
                    const int g = rr / hd;
                    __half2* dst = (__half2*)(a.kcache + (int64_t)s * a.kv_seq_stride +
                                              ((int64_t)g * a.max_ctx + p) * hd + (rr % hd));
                    *dst = __floats2half2_rn(z0, z1);
                }
            } else {
                const int rr = r0 - a.q_rows - a.kv_rows;
                const int g = rr / hd;
                __half2* dst = (__half2*)(a.vcache + (int64_t)s * a.kv_seq_stride +
                                          ((int64_t)g * a.max_ctx + p) * hd + (rr % hd));
                *dst = __floats2half2_rn(y0, y1);
            }
        } else if (EPI == EPI_RESID) {
            float* xo = a.out + (int64_t)s * a.out_stride + r0;
            float2 v = *(float2*)xo;
            v.x += y0;
            v.y += y1;
            *(float2*)xo = v;
        } else if (EPI == EPI_SWIGLU) {
            // row 2i = gate i, row 2i+1 = up i: h_i = silu(gate) * up
            const float sg = y0 / (1.0f + __expf(-y0));
            a.out[(int64_t)s * a.out_stride + (r0 >> 1)] = sg * y1;
        } else {  // EPI_LOGITS
            if (a.out) *(float2*)(a.out + (int64_t)s * a.out_stride + r0) = make_float2(y0, y1);
            better(best_v, best_i, y0, r0);
            better(best_v, best_i, y1, r0 + 1);
        }
    };

    // ---- prologue.  RMSNorm(x) * g = s * (x . g) with the scalar
    // s = 1/sqrt(mean(x^2) + eps): x . g is staged into LDS and s multiplies
    // each row's finished dot product, so no element waits for the reduction.
    // The first x batch is requested before the first weight chunk; in-order
    // load counters then let it be consumed while the weights are in flight.
    constexpr int kXr = 4;                       // float4s per thread per batch
    float4 xr[kXr], gr[kXr];
    const bool has_g = a.norm_g != nullptr;
    #pragma unroll
    for (int u = 0; u < kXr; ++u) {
        const int i = min((tid + u * kBlock) * 4, K - 4);
        xr[u] = *(const float4*)(x + i);
        if (has_g) gr[u] = *(const float4*)(a.norm_g + i);
    }
    WChunk<QT> wa, wb;
    load(0, wa);          // unconditional: rows are clamped, so this is always in bounds

    float ss = 0.f;
    for (int base = 0; base < K; base += kXr * kBlock * 4) {
        if (base > 0) {
            #pragma unroll
            for (int u = 0; u < kXr; ++u) {
                const int i = min(base + (tid + u * kBlock) * 4, K - 4);
                xr[u] = *(const float4*)(x + i);
                if (has_g) gr[u] = *(const float4*)(a.norm_g + i);
            }
        }
        #pragma unroll
        for (int u = 0; u < kXr; ++u) {
            const int i = base + (tid + u * kBlock) * 4;
            if (i < K) {
                float4 v = xr[u];
                if (has_g) {
                    ss = fmaf(v.x, v.x, ss);
                    ss = fmaf(v.y, v.y, ss);
                    ss = fmaf(v.z, v.z, ss);
                    ss = fmaf(v.w, v.w, ss);
                    v.x *= gr[u].x;
                    v.y *= gr[u].y;
                    v.z *= gr[u].z;
                    v.w *= gr[u].w;
                }
                *(float4*)(xs + xswz(i)) = v;
            }
        }
    }
    // block_sum's barriers also order the LDS stores above before any reads
    if (has_g) rscale = 1.0f / sqrtf(block_sum(ss, red) / (float)K + a.eps);
    __syncthreads();
    if (QT == kQ4_0) {
        for (int b = tid; b < nb; b += kBlock) {
            const float* xb = xs + (b << 5);
            float t = 0.f;
            #pragma unroll
            for (int e = 0; e < 32; ++e) t += xb[e];
            bsum[b] = t;
        }
        __syncthreads();
    }

    // ---- two-stage pipeline: chunk c+1's loads are in flight while c computes.
    // The steady-state body issues its loads unconditionally (exact load
    // counters); the last one or two chunks are peeled off.
    int c = 0;
    for (; c + 2 < n_chunks; c += 2) {
        load(c + 1, wb);
        compute(c, wa);
        finish(c);
        load(c + 2, wa);
        compute(c + 1, wb);
        finish(c + 1);
    }
    if (c + 1 < n_chunks) {
        load(c + 1, wb);
        compute(c, wa);
        finish(c);
        compute(c + 1, wb);
        finish(c + 1);
    } else if (c < n_chunks) {
        compute(c, wa);
        finish(c);
    }

    if (EPI == EPI_LOGITS) {
        // workgroup maximum, then the last workgroup of the sequence reduces
        #pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(best_v, off, 64);
            const int oi = __shfl_xor(best_i, off, 64);
            better(best_v, best_i, ov, oi);
        }
        if (lane == 0) { wv_best[wave] = best_v; wi_best[wave] = best_i; }
        __syncthreads();
        if (tid == 0) {
            float bv = wv_best[0];
            int bi = wi_best[0];
            for (int w = 1; w < kWaves; ++w) better(bv, bi, wv_best[w], wi_best[w]);
            a.part_val[(int64_t)s * gridDim.x + blockIdx.x] = bv;
            a.part_idx[(int64_t)s * gridDim.x + blockIdx.x] = bi;
            __threadfence();
            const int old = atomicAdd(&a.counter[s], 1);
            s_last = (old == (int)gridDim.x - 1);
        }
        __syncthreads();
        if (s_last) {
            if (tid == 0) __threadfence();
            __syncthreads();
            float bv = -FLT_MAX;
            int bi = INT_MAX;
            for (int i = tid; i < (int)gridDim.x; i += kBlock)
                better(bv, bi, a.part_val[(int64_t)s * gridDim.x + i],
                       a.part_idx[(int64_t)s * gridDim.x + i]);
            #pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const float ov = __shfl_xor(bv, off, 64);
                const int oi = __shfl_xor(bi, off, 64);
                better(bv, bi, ov, oi);
            }
            if (lane == 0) { wv_best[wave] = bv; wi_best[wave] = bi; }
            __syncthreads();
            if (tid == 0) {
                for (int w = 1; w < kWaves; ++w) better(wv_best[0], wi_best[0], wv_best[w], wi_best[w]);
                a.argmax_out[s] = wi_best[0];
                if (a.pos_inc) a.pos_inc[s] += 1;
                a.counter[s] = 0;
            }
        }
    }
}

static int pick_lpr(int nb) {
    if (nb >= 64) return 64;
    if (nb >= 32) return 32;
    if (nb >= 16) return 16;
    return 8;
}

template <int QT, int LPR, int EPI>
static int resident_blocks(size_t lds) {
    // workgroups of this instantiation that fit on the whole device at once
    static int cached_cus = 0;
    if (!cached_cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cached_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cached_cus = 256;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_gemv<QT, LPR, EPI>, kBlock, lds) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return per_cu * cached_cus;
}

template <int QT, int LPR, int EPI>
static hipError_t launch_one(const GemvArgs& a, int n_seq, int max_blocks, size_t lds, hipStream_t st) {
    constexpr int rows_per_step = 2 * (64 / LPR);
    const int n_steps = (a.w.N + rows_per_step - 1) / rows_per_step;
    int g = (n_steps + kWaves - 1) / kWaves;
    const int cap = std::min(max_blocks, resident_blocks<QT, LPR, EPI>(lds));
    if (g > cap) {
        // equal work per workgroup: the fewest blocks that keep the grid-stride rounds balanced
        const int rounds = (g + cap - 1) / cap;
        g = (g + rounds - 1) / rounds;
    }
    if (g < 1) g = 1;
    hipLaunchKernelGGL((k_gemv<QT, LPR, EPI>), dim3(g, n_seq), dim3(kBlock), lds, st, a);
    return hipGetLastError();
}

template <int QT, int EPI>
static hipError_t launch_gemv_lpr(const GemvArgs& a, int lpr, int n_seq, int max_blocks, size_t lds,
                                  hipStream_t st) {
    switch (lpr) {
        case 64: return launch_one<QT, 64, EPI>(a, n_seq, max_blocks, lds, st);
        case 32: return launch_one<QT, 32, EPI>(a, n_seq, max_blocks, lds, st);
        case 16: return launch_one<QT, 16, EPI>(a, n_seq, max_blocks, lds, st);
        default: return launch_one<QT, 8, EPI>(a, n_seq, max_blocks, lds, st);
    }
}

template <int QT>
static hipError_t launch_gemv_epi(const GemvArgs& a, int epi, int lpr, int n_seq, int max_blocks, size_t lds,
                                  hipStream_t st) {
    switch (epi) {
        case EPI_QKV: return launch_gemv_lpr<QT, EPI_QKV>(a, lpr, n_seq, max_blocks, lds, st);
        case EPI_RESID: return launch_gemv_lpr<QT, EPI_RESID>(a, lpr, n_seq, max_blocks, lds, st);
        case EPI_SWIGLU: return launch_gemv_lpr<QT, EPI_SWIGLU>(a, lpr, n_seq, max_blocks, lds, st);
        default: return launch_gemv_lpr<QT, EPI_LOGITS>(a, lpr, n_seq, max_blocks, lds, st);
    }
}

hipError_t launch_gemv(const GemvArgs& a, int epi, int n_seq, int max_blocks, hipStream_t st) {
    const int nb = a.w.K / 32;
    const int lpr = pick_lpr(nb);
    const size_t lds = (size_t)(a.w.K + (a.qtype == kQ4_0 ? nb : 0)) * sizeof(float);
    if (a.qtype == kQ8_0) return launch_gemv_epi<kQ8_0>(a, epi, lpr, n_seq, max_blocks, lds, st);
    return launch_gemv_epi<kQ4_0>(a, epi, lpr, n_seq, max_blocks, lds, st);
}

// ---------------------------------------------------------------------------
// GQA decode attention, split over context, combined by the last workgroup
// ---------------------------------------------------------------------------
constexpr int kMaxGroup = 8;   // query heads per KV head

template <int HD>
__global__ __launch_bounds__(kBlock) void k_attn(AttnArgs a) {
    constexpr int CH = kAttnChunk;
    __shared__ __align__(16) __half Ks[CH][HD + 2];   // +2 halves: row stride of an odd word count
    __shared__ __align__(16) __half Vs[CH][HD];
    __shared__ __align__(16) float Qs[kMaxGroup][HD];
    __shared__ __align__(16) float Ps[kMaxGroup][CH];
    __shared__ int s_last;

    const int chunk = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = a.nq / a.nkv;
    const int n_ctx = a.pos[s] + 1;                 // keys 0..pos inclusive
    const int t0 = chunk * CH;
    const int64_t stride = HD + 2;
    float* part_s = a.part + (int64_t)s * a.nq * a.max_chunks * stride;

    if (t0 < n_ctx) {
        const int nt = min(CH, n_ctx - t0);
        const __half* Kg = a.kcache + (int64_t)s * a.kv_seq_stride + ((int64_t)g * a.max_ctx + t0) * HD;
        const __half* Vg = a.vcache + (int64_t)s * a.kv_seq_stride + ((int64_t)g * a.max_ctx + t0) * HD;
        // every 16-byte load of the tile (and q) is issued before any is used
        constexpr int kPer = CH * (HD / 8) / kBlock;     // 16-byte pieces per thread
        uint4 kr[kPer], vr[kPer];
        #pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int c = tid + u * kBlock;
            const int t = c / (HD / 8), d8 = (c % (HD / 8)) * 8;
            if (t < nt) {
                kr[u] = *(const uint4*)(Kg + (int64_t)t * HD + d8);
                vr[u] = *(const uint4*)(Vg + (int64_t)t * HD + d8);
            }
        }
        const float* qg = a.q + (int64_t)s * a.nq * HD + (int64_t)g * G * HD;
        float qv[kMaxGroup * HD / kBlock];
        #pragma unroll
        for (int u = 0; u < kMaxGroup * HD / kBlock; ++u) {
            const int i = tid + u * kBlock;
            if (i < G * HD) qv[u] = qg[i];
        }
        #pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int c = tid + u * kBlock;
            const int t = c / (HD / 8), d8 = (c % (HD / 8)) * 8;
            if (t < nt) {
                uint32_t* kd = (uint32_t*)&Ks[t][d8];
                kd[0] = kr[u].x; kd[1] = kr[u].y; kd[2] = kr[u].z; kd[3] = kr[u].w;
                *(uint4*)&Vs[t][d8] = vr[u];
            }
        }
        #pragma unroll
        for (int u = 0; u < kMaxGroup * HD / kBlock; ++u) {
            const int i = tid + u * kBlock;
            if (i < G * HD) Qs[i / HD][i % HD] = qv[u];
        }
        __syncthreads();

        // scores and the chunk's softmax state, one head per wavefront pass
        for (int j = wave; j < G; j += kWaves) {
            float sc = -FLT_MAX;
            if (lane < nt) {
                float acc0 = 0.f, acc1 = 0.f;
                #pragma unroll 8
                for (int d = 0; d < HD; d += 2) {
                    const float2 kk = __half22float2(*(const __half2*)&Ks[lane][d]);
                    acc0 = fmaf(Qs[j][d], kk.x, acc0);
                    acc1 = fmaf(Qs[j][d + 1], kk.y, acc1);
                }
                sc = (acc0 + acc1) * a.scale;
            }
            const float m = wave_max(sc);
            const float p = lane < nt ? __expf(sc - m) : 0.f;
            const float l = wave_sum(p);
            Ps[j][lane] = p;
            if (lane == 0) {
                float* ph = part_s + ((int64_t)(g * G + j) * a.max_chunks + chunk) * stride;
                ph[HD] = m;
                ph[HD + 1] = l;
            }
        }
        __syncthreads();
        for (int i = tid; i < G * HD; i += kBlock) {
            const int j = i / HD, d = i % HD;
            float o0 = 0.f, o1 = 0.f;
            int t = 0;
            for (; t + 1 < nt; t += 2) {
                o0 = fmaf(Ps[j][t], __half2float(Vs[t][d]), o0);
                o1 = fmaf(Ps[j][t + 1], __half2float(Vs[t + 1][d]), o1);
            }
            if (t < nt) o0 = fmaf(Ps[j][t], __half2float(Vs[t][d]), o0);
            part_s[((int64_t)(g * G + j) * a.max_chunks + chunk) * stride + d] = o0 + o1;
        }
    }

    // completion count; the last workgroup of (s, g) merges the chunks.  The
    // barrier completes every thread's stores; one agent-scope fence per
    // workgroup then publishes them before the counter moves.
    __syncthreads();
    if (tid == 0) {
        __threadfence();
        const int old = atomicAdd(&a.counter[s * a.nkv + g], 1);
        s_last = (old == (int)gridDim.x - 1);
    }
    __syncthreads();
    if (!s_last) return;
    if (tid == 0) __threadfence();
    __syncthreads();
    const int n_act = (n_ctx + CH - 1) / CH;
    for (int i = tid; i < G * HD; i += kBlock) {
        const int j = i / HD, d = i % HD;
        const int h = g * G + j;
        const float* ph = part_s + (int64_t)h * a.max_chunks * stride;
        // one pass with running rescaling: (M, L, O) merge chunk by chunk
        float M = -FLT_MAX, L = 0.f, O = 0.f;
        for (int c = 0; c < n_act; ++c) {
            const float mc = ph[c * stride + HD];
            const float lc = ph[c * stride + HD + 1];
            const float oc = ph[c * stride + d];
            const float Mn = fmaxf(M, mc);
            const float r = __expf(M - Mn), e = __expf(mc - Mn);
            L = fmaf(L, r, lc * e);
            O = fmaf(O, r, oc * e);
            M = Mn;
        }
        a.out[(int64_t)s * a.nq * HD + (int64_t)h * HD + d] = O / L;
    }
    if (tid == 0) a.counter[s * a.nkv + g] = 0;
}

hipError_t launch_attention(const AttnArgs& a, int n_seq, hipStream_t st) {
    dim3 grid(a.max_chunks, a.nkv, n_seq);
    if (a.hd == 128) hipLaunchKernelGGL(k_attn<128>, grid, dim3(kBlock), 0, st, a);
    else if (a.hd == 64) hipLaunchKernelGGL(k_attn<64>, grid, dim3(kBlock), 0, st, a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// inspection kernels
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_dequant(QMat w, int qtype, int row0, float* __restrict__ out) {
    const int r = row0 + blockIdx.x;
    const int K = w.K, nb = K >> 5;
    const int64_t rowq = qtype == kQ8_0 ? (int64_t)K : (int64_t)(K >> 1);
    const uint8_t* q = w.q + (int64_t)r * rowq;
    for (int c = threadIdx.x; c < K; c += kBlock) {
        const int b = c >> 5, e = c & 31;
        const float d = h2f(w.sc[(int64_t)r * nb + b]);
        float v;
        if (qtype == kQ8_0) {
            const int8_t qi = (int8_t)(e < 16 ? q[b * 16 + e] : q[(int64_t)nb * 16 + b * 16 + (e - 16)]);
            v = d * (float)qi;
        } else {
            const uint8_t byte = q[b * 16 + (e & 15)];
            const int nib = e < 16 ? (byte & 0xF) : (byte >> 4);
            v = (float)(nib - 8) * d;
        }
        out[(int64_t)blockIdx.x * K + c] = v;
    }
}

hipError_t launch_dequant(const QMat& w, int qtype, int row0, int n_rows, float* out, hipStream_t st) {
    hipLaunchKernelGGL(k_dequant, dim3(n_rows), dim3(kBlock), 0, st, w, qtype, row0, out);
    return hipGetLastError();
}

__global__ __launch_bounds__(kBlock) void k_read_bw(const uint4* __restrict__ buf, int64_t n16,
                                                   float* __restrict__ sink) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n16; i += stride) {
        const uint4 v = buf[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    acc = (uint32_t)wave_sum((float)(acc & 0xFFFF));
    if (threadIdx.x == 0) sink[blockIdx.x] = (float)acc;
}

hipError_t launch_read_bw(const void* buf, int64_t n_bytes, float* sink, hipStream_t st) {
    hipLaunchKernelGGL(k_read_bw, dim3(2048), dim3(kBlock), 0, st, (const uint4*)buf, n_bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace lmk
