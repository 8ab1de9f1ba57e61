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
//  * one-sequence dequant-GEMV: one workgroup per CU stages the input as
//    24-bit integer digits in LDS (its RMSNorm folded in); a wavefront owns
//    two adjacent output rows at a time (so a RoPE pair or a gate/up pair
//    ends in the same lanes) and its lanes split the row's blocks; quants
//    arrive as coalesced 16-byte loads from the repacked half-block planes,
//    v_dot4_i32_i8 gives each digit plane's exact int32 block sum, fp32
//    accumulation, row sums by DPP moves and row/half-wave swaps.  RoPE +
//    fp16 KV append, SwiGLU, residual add, or logits + argmax run in the
//    epilogue.
//  * 2-4 sequences: the same digits as the first operand of the int8 matrix
//    core (v_mfma_i32_16x16x32_i8), the weights' fragment copy as the second.
//  * attention: one workgroup per (span of 64-position tiles, KV head,
//    sequence) scores all query heads of the group on the matrix cores, each
//    wavefront keeping its own online softmax; the last workgroup of a
//    (sequence, KV head) to finish merges the spans' partial softmax states
//    (log-sum-exp) - no second launch.
#include "lm_internal.h"
#include "lm_device.h"

#include <float.h>
#include <limits.h>

#include <algorithm>
#include <mutex>

namespace lmk {

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

// Weight blocks one lane loads per pipeline stage (per row of its row pair).
template <int QT> struct ChunkBlocks { static constexpr int value = LMK_CB_Q8; };
template <> struct ChunkBlocks<kQ4_0> { static constexpr int value = LMK_CB_Q4; };
template <> struct ChunkBlocks<kQ4_K> { static constexpr int value = LMK_CB_QK; };
template <> struct ChunkBlocks<kQ5_K> { static constexpr int value = LMK_CB_QK; };
template <> struct ChunkBlocks<kQ6_K> { static constexpr int value = LMK_CB_QK; };

// One pipeline stage of a lane: CB blocks of both rows of its row pair.
template <int QT>
struct WChunk {
    static constexpr int CB = ChunkBlocks<QT>::value;
    int4 a0[CB], a1[CB];          // first 16 bytes (Q8_0) / the 16 nibble bytes (others) of row 0 / row 1
    int4 b0[QT == kQ8_0 ? CB : 1], b1[QT == kQ8_0 ? CB : 1];   // Q8_0 second halves
    static constexpr bool kHdr = QT == kQ4_K || QT == kQ5_K;
    int4 h0[kHdr ? CB : 1], h1[kHdr ? CB : 1];                 // Q4_K / Q5_K super-block headers
    uint32_t p0[QT == kQ5_K ? CB : 1], p1[QT == kQ5_K ? CB : 1];   // Q5_K fifth bits
    uint2 e0[QT == kQ6_K ? CB : 1], e1[QT == kQ6_K ? CB : 1];  // Q6_K high bits
    static constexpr bool kPair = (QT == kQ8_0 || QT == kQ4_0) && kScPairs;
    uint16_t d0[kPair ? 1 : CB], d1[kPair ? 1 : CB];   // block scales of row 0 / 1 (Q8_0, Q4_0) or the
                                                       // sub-block scale pairs (Q6_K)
    uint32_t dd[kPair ? CB : 1];   // Q8_0 / Q4_0 with paired scales: both rows' block scale (row 0 low)
    uint16_t f0[QT == kQ6_K ? CB : 1], f1[QT == kQ6_K ? CB : 1];   // Q6_K super-block d
};

#ifndef LMK_GEMV_MIN_BLOCKS
#define LMK_GEMV_MIN_BLOCKS 1     // workgroups per CU the register budget must allow
#endif

// XR: float4s of the input each thread requests per prologue batch (2, 4 or
// 8: K up to 4096, 8192 or 16384 columns in one round trip with 512 threads);
// a template parameter so the register budget of the short-K kernels stays
// small.
// NT threads per workgroup, one workgroup per CU (the input staged once per
// CU): 512 by default; 256, 768 or 1024 for a matrix whose row pairs fill the
// chip in one round of that many wavefronts (launch_wide_rows); the LM head
// 256 (about 60 row pairs per wavefront; measured faster than 512).
template <int QT, int LPR, int EPI, int XR, int NT, bool WNT>
__global__ __launch_bounds__(NT, LMK_GEMV_MIN_BLOCKS) void k_gemv(GemvArgs a) {
    constexpr int NW = NT / 64;
    extern __shared__ __align__(16) float smem[];
    __shared__ float red[NW];
    __shared__ float wv_best[NW];
    __shared__ int wi_best[NW];
    __shared__ int s_last;

    constexpr int CB = ChunkBlocks<QT>::value;
    constexpr int kGroups = 64 / LPR;            // row pairs per wavefront step
    constexpr int kRowsPerStep = 2 * kGroups;

    const int K = a.w.K, N = a.w.N, nb = K >> 5;
    // LDS: per 32-column block, the activation digit planes (96 bytes), its
    // scale, and the digit sums (Q4_0, Q4_K: per block; Q6_K: per 16-column half)
    constexpr int kSums = (QT == kQ4_0 || QT == kQ4_K || QT == kQ5_K) ? 1 : (QT == kQ6_K ? 2 : 0);
    int8_t* xq = (int8_t*)smem;                       // [nb][3][32] int8
    float* xsc = (float*)(xq + nb * 96);              // [nb]
    int4* dsum = (int4*)(xsc + ((nb + 3) & ~3));      // [nb or 2 nb] (T0, T1, T2, 0)
    const int tid = threadIdx.x, lane = tid & 63;
    // wave-uniform by construction; readfirstlane lets the row bases live in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = blockIdx.y;
    const float* x = a.xin + (int64_t)s * a.x_stride;
    const int rg = lane / LPR, li = lane % LPR;
    const int64_t rowq = qmat_qbytes(QT, 1, K);
    // scale-plane row in 16-bit words (layouts in lm_internal.h)
    const int srow = (int)(qmat_srow(QT, K) / 2);
    static_assert(LPR % 8 == 0, "a lane's blocks must share their position in the 8-block super-block");
    const int jsub = li & 7;   // Q4_K: sub-block of every block this lane reads

    // this wavefront's steps: step0, step0 + sstride, ... ; each step is split
    // into `cps` chunks of CB blocks per lane
    const int n_steps = (N + kRowsPerStep - 1) / kRowsPerStep;
    // (dealt round-robin over the workgroups first, so every CU holds an equal
    // share, within one, whatever the number of steps)
    const int step0 = wave * (int)gridDim.x + (int)blockIdx.x, sstride = gridDim.x * NW;
    const int my_steps = step0 < n_steps ? (n_steps - 1 - step0) / sstride + 1 : 0;
    const int bpl = (nb + LPR - 1) / LPR;        // blocks per lane per row (upper bound)
    const int cps = (bpl + CB - 1) / CB;
    const int n_chunks = my_steps * cps;

    int rope_p = 0;                       // the position (read after the weight requests)
    float pre_cs = 1.f, pre_sn = 0.f;     // RoPE cos/sin of the first row pair (below)
    float2 pre_res = make_float2(0.f, 0.f);   // residual of the first row pair (below)

    // Branch-free loads (clamped addresses; a block past the row end gets
    // scale 0) so the compiler's in-order load counters stay exact and the
    // next chunk's loads remain in flight while this one computes.
    auto load = [&](int c, WChunk<QT>& w) {
        const int i = c / cps, k = c - i * cps;
        const int r0 = min((step0 + i * sstride) * kRowsPerStep + rg * 2, N - 2);
        const uint8_t* q0 = a.w.q + (int64_t)r0 * rowq;
        const uint8_t* q1 = q0 + rowq;
        // Q8_0 / Q4_0: the row pair's scales interleaved, (row r0, row r0+1) per block
        const uint16_t* s0 = a.w.sc + (int64_t)r0 * srow;
        #pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int b = li + LPR * (k * CB + u);
            const uint32_t bc = (uint32_t)min(b, nb - 1);   // unsigned 32-bit offsets: scalar base + vector offset
            w.a0[u] = ld16_w<WNT>(q0 + bc * 16u);
            w.a1[u] = ld16_w<WNT>(q1 + bc * 16u);
            if (QT == kQ8_0) {
                w.b0[u] = ld16_w<WNT>(q0 + (uint32_t)nb * 16u + bc * 16u);
                w.b1[u] = ld16_w<WNT>(q1 + (uint32_t)nb * 16u + bc * 16u);
            }
            if (QT == kQ4_K || QT == kQ5_K) {
                w.h0[u] = ld16_stream((const uint8_t*)(s0 + (bc >> 3) * 8u));
                w.h1[u] = ld16_stream((const uint8_t*)(s0 + (uint32_t)srow + (bc >> 3) * 8u));
                if (QT == kQ5_K) {
                    w.p0[u] = ld4_stream(q0 + (uint32_t)nb * 16u + bc * 4u);
                    w.p1[u] = ld4_stream(q1 + (uint32_t)nb * 16u + bc * 4u);
                }
            } else if (QT == kQ6_K) {
                w.e0[u] = ld8_stream(q0 + (uint32_t)nb * 16u + bc * 8u);
                w.e1[u] = ld8_stream(q1 + (uint32_t)nb * 16u + bc * 8u);
                w.d0[u] = s0[bc];
                w.d1[u] = s0[(uint32_t)srow + bc];
                w.f0[u] = s0[(uint32_t)nb + (bc >> 3)];
                w.f1[u] = s0[(uint32_t)(srow + nb) + (bc >> 3)];
            } else if (WChunk<QT>::kPair) {
                // both rows' block scales in one 32-bit load; consumed only in compute():
                // consuming a load here would wait on every load issued before it
                w.dd[u] = ld4_w<WNT>(s0 + bc * 2u);
            } else {
                w.d0[u] = s0[bc];
                w.d1[u] = s0[(uint32_t)srow + bc];
            }
        }
    };

    float acc0 = 0.f, acc1 = 0.f;
    auto compute = [&](int c, const WChunk<QT>& w) {
        const int k = c % cps;
        #pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int braw = li + LPR * (k * CB + u);
            const int b = min(braw, nb - 1);
            const bool in_row = braw < nb;                     // past the row end: no contribution
            const int4* D = (const int4*)(xq + b * 96);
            const float sx = xsc[b];
            const uint16_t h0 = WChunk<QT>::kPair ? (uint16_t)(w.dd[u] & 0xFFFFu) : w.d0[u];
            const uint16_t h1 = WChunk<QT>::kPair ? (uint16_t)(w.dd[u] >> 16) : w.d1[u];
            if (QT == kQ8_0) {
                const float d0 = in_row ? h2f(h0) : 0.f;
                const float d1 = in_row ? h2f(h1) : 0.f;
                acc0 = fmaf(d0 * sx, dot_q8(w.a0[u], w.b0[u], D), acc0);
                acc1 = fmaf(d1 * sx, dot_q8(w.a1[u], w.b1[u], D), acc1);
            } else if (QT == kQ4_0) {
                const float d0 = in_row ? h2f(h0) : 0.f;
                const float d1 = in_row ? h2f(h1) : 0.f;
                const int4 T = dsum[b];
                acc0 = fmaf(d0 * sx, dot_q4(w.a0[u], D, T), acc0);
                acc1 = fmaf(d1 * sx, dot_q4(w.a1[u], D, T), acc1);
            } else if (QT == kQ4_K || QT == kQ5_K) {
                // sum (ds q - dm) x = ds sum q x - dm sum x over the sub-block
                float ds0, dm0, ds1, dm1;
                q4k_scale_min(w.h0[u], jsub, ds0, dm0);
                q4k_scale_min(w.h1[u], jsub, ds1, dm1);
                const float f = in_row ? sx : 0.f;
                const int4 T = dsum[b];
                const float tx = combine_digits(T.x, T.y, T.z);
                const float q0x = QT == kQ5_K ? dot_q5(w.a0[u], w.p0[u], D) : dot_q4<0>(w.a0[u], D, T);
                const float q1x = QT == kQ5_K ? dot_q5(w.a1[u], w.p1[u], D) : dot_q4<0>(w.a1[u], D, T);
                acc0 = fmaf(ds0 * f, q0x, acc0);
                acc0 = fmaf(-dm0 * f, tx, acc0);
                acc1 = fmaf(ds1 * f, q1x, acc1);
                acc1 = fmaf(-dm1 * f, tx, acc1);
            } else {  // Q6_K
                const int4 T0 = dsum[2 * b], T1 = dsum[2 * b + 1];
                float lo0, hi0, lo1, hi1;
                dot_q6(w.a0[u], w.e0[u], D, T0, T1, lo0, hi0);
                dot_q6(w.a1[u], w.e1[u], D, T0, T1, lo1, hi1);
                const float g0 = in_row ? h2f(w.f0[u]) * sx : 0.f, g1 = in_row ? h2f(w.f1[u]) * sx : 0.f;
                const float c00 = (float)(int8_t)(w.d0[u] & 255), c01 = (float)(int8_t)(w.d0[u] >> 8);
                const float c10 = (float)(int8_t)(w.d1[u] & 255), c11 = (float)(int8_t)(w.d1[u] >> 8);
                acc0 = fmaf(g0, fmaf(c00, lo0, c01 * hi0), acc0);
                acc1 = fmaf(g1, fmaf(c10, lo1, c11 * hi1), acc1);
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
        acc0 = group_sum<LPR>(acc0);
        acc1 = group_sum<LPR>(acc1);
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
            float2 v = i == 0 ? pre_res : *(float2*)xo;
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
    // The x batch is requested before the first weight chunks (XR float4s
    // per thread, chosen from K at launch); in-order load counters let it be
    // consumed while the weights are still in flight.  The residual
    // projections (Wo, down) take no gain.
    constexpr bool kGain = EPI != EPI_RESID;
    constexpr int GR = kGain ? XR : 1;
    const bool has_g = kGain && a.norm_g != nullptr;
    float4 xr[XR], gr[GR];
    auto fetch = [&](int base) {
        #pragma unroll
        for (int u = 0; u < XR; ++u) {
            const int i = min(base + (tid + u * NT) * 4, K - 4);
            xr[u] = *(const float4*)(x + i);
            if (kGain && has_g) gr[u % GR] = *(const float4*)(a.norm_g + i);
        }
    };
    fetch(0);
    // keep the input loads ahead of the weight loads: the in-order counters
    // then release x while the weights are still arriving
    __builtin_amdgcn_sched_barrier(0);
    WChunk<QT> wa, wb;
    load(0, wa);          // unconditional: rows are clamped, so these are always in bounds
    load(1, wb);
    float ss = 0.f;
    for (int base = 0; base < K; base += XR * NT * 4) {
        if (base > 0) fetch(base);
        #pragma unroll
        for (int u = 0; u < XR; ++u) {
            // the 8 threads tid..tid|7 hold one 32-column block (K % 32 == 0, so a
            // block is either wholly inside K or wholly past it: uniform per group)
            const int i = base + (tid + u * NT) * 4;
            float4 v = xr[u];
            if (kGain && has_g) {
                if (i < K) {
                    ss = fmaf(v.x, v.x, ss);
                    ss = fmaf(v.y, v.y, ss);
                    ss = fmaf(v.z, v.z, ss);
                    ss = fmaf(v.w, v.w, ss);
                }
                const float4 gv = gr[u % GR];
                v.x *= gv.x;
                v.y *= gv.y;
                v.z *= gv.z;
                v.w *= gv.w;
            }
            stage_digits(v, i, K, xq, xsc, dsum, kSums);
        }
    }
    // block_sum's barriers also order the LDS stores above before any reads
    if (has_g) rscale = 1.0f / sqrtf(block_sum<NW>(ss, red) / (float)K + a.eps);
    __syncthreads();

    // ---- the position and the RoPE inputs of this wavefront's first row pair.
    // Requested only now, behind the weights: the position is a scalar load,
    // and scalar loads are waited for all together, so reading it before the
    // weight requests would hold the whole stream for its round trip.  The
    // table loads are unconditional (clamped row): exact load counters.
    if (EPI == EPI_QKV) {
        rope_p = a.pos[s];
        const int r0 = min(step0 * kRowsPerStep + rg * 2, a.q_rows + a.kv_rows - 2);
        const int rr = r0 < a.q_rows ? r0 : r0 - a.q_rows;
        const int pi = (rr % a.head_dim) >> 1;
        pre_cs = a.rope_cos[(int64_t)rope_p * (a.head_dim >> 1) + pi];
        pre_sn = a.rope_sin[(int64_t)rope_p * (a.head_dim >> 1) + pi];
    }
    // the residual the first row pair adds to, likewise behind the weights
    // (only this row pair's lanes write it, after the read).  A vector load:
    // the address is uniform, and a scalar load in flight would make the
    // main loop's LDS waits wait for it too.
    if (EPI == EPI_RESID) {
        int vzero;
        asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
        const int r0 = min(step0 * kRowsPerStep + rg * 2, N - 2) + vzero;
        pre_res = *(const float2*)(a.out + (int64_t)s * a.out_stride + r0);
    }

    // ---- pipeline: a chunk's registers are refilled (chunk c+2) as soon as
    // chunk c has been consumed, before c's cross-lane reduction and
    // epilogue, so two chunks stay in flight.  The steady-state body issues
    // its loads unconditionally (exact load counters); the tail is peeled.
    int c = 0;
    for (; c + 3 < n_chunks; c += 2) {
        compute(c, wa);
        load(c + 2, wa);
        finish(c);
        compute(c + 1, wb);
        load(c + 3, wb);
        finish(c + 1);
    }
    // at most three chunks left: c (in wa), c+1 (in wb), c+2 (not loaded)
    if (c < n_chunks) {
        compute(c, wa);
        if (c + 2 < n_chunks) load(c + 2, wa);
        finish(c);
    }
    if (c + 1 < n_chunks) {
        compute(c + 1, wb);
        finish(c + 1);
    }
    if (c + 2 < n_chunks) {
        compute(c + 2, wa);
        finish(c + 2);
    }
    if (EPI == EPI_LOGITS) {
        // workgroup maximum, then the last workgroup of the sequence reduces
        group_argmax<64>(best_v, best_i);
        if (lane == 0) { wv_best[wave] = best_v; wi_best[wave] = best_i; }
        __syncthreads();
        if (tid == 0) {
            float bv = wv_best[0];
            int bi = wi_best[0];
            for (int w = 1; w < NW; ++w) better(bv, bi, wv_best[w], wi_best[w]);
            // the workgroup's candidate, handed to the last workgroup as the
            // attention chunks hand over their states (lm_device.h)
            st_dev(&a.part_val[(int64_t)s * gridDim.x + blockIdx.x], bv);
            st_dev(&a.part_idx[(int64_t)s * gridDim.x + blockIdx.x], bi);
            drain_vm();
            s_last = count_arrive(&a.counter[s], (int)gridDim.x);
        }
        __syncthreads();
        if (s_last) {
            float bv = -FLT_MAX;
            int bi = INT_MAX;
            for (int i = tid; i < (int)gridDim.x; i += NT)
                better(bv, bi, ld_dev(&a.part_val[(int64_t)s * gridDim.x + i]),
                       ld_dev(&a.part_idx[(int64_t)s * gridDim.x + i]));
            group_argmax<64>(bv, bi);
            if (lane == 0) { wv_best[wave] = bv; wi_best[wave] = bi; }
            __syncthreads();
            if (tid == 0) {
                for (int w = 1; w < NW; ++w) better(wv_best[0], wi_best[0], wv_best[w], wi_best[w]);
                a.argmax_out[s] = wi_best[0];
                if (a.pos_inc) a.pos_inc[s] += 1;
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

static int device_cus() {
    static int cached_cus = 0;
    if (!cached_cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cached_cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cached_cus = 256;
    }
    return cached_cus;
}

#ifndef LMK_LMHEAD_NT
#define LMK_LMHEAD_NT 256
#endif
#ifndef LMK_GEMV_WPC
#define LMK_GEMV_WPC 1      // workgroups per CU
#endif
template <int EPI> constexpr int gemv_threads() { return EPI == EPI_LOGITS ? LMK_LMHEAD_NT : kGemvThreads; }

template <int QT, int LPR, int EPI, int XR, int NT = gemv_threads<EPI>()>
static hipError_t launch_one(const GemvArgs& a, int n_seq, int max_blocks, size_t lds, hipStream_t st) {
    constexpr int rows_per_step = 2 * (64 / LPR);
    constexpr int nw = NT / 64;
    const int n_steps = (a.w.N + rows_per_step - 1) / rows_per_step;
    (void)nw;
    // One workgroup per CU (NT / 64 wavefronts: eight measured best for a
    // long GEMV on gfx950); a longer matrix takes several row-pair rounds
    // per wavefront.
    int g = std::min({n_steps, device_cus() * LMK_GEMV_WPC, max_blocks});
    if (g < 1) g = 1;
    // the non-temporal hint for large matrices only (lm_device.h); the K
    // formats take it at every size
    if constexpr (QT == kQ8_0 || QT == kQ4_0) {
        if ((int64_t)a.w.N * qmat_qbytes(QT, 1, a.w.K) < kStreamBytes) {
            hipLaunchKernelGGL((k_gemv<QT, LPR, EPI, XR, NT, false>), dim3(g, n_seq), dim3(NT), lds, st, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_gemv<QT, LPR, EPI, XR, NT, true>), dim3(g, n_seq), dim3(NT), lds, st, a);
    return hipGetLastError();
}

// A matrix whose row-pair steps fill every CU in one round of 4 to 16
// wavefronts takes a workgroup of exactly that many wavefronts per CU (each
// wavefront one step, the whole matrix in flight at once); others keep eight
// wavefronts and take several rounds.  XR covers K in one input batch where
// it can (the prologue loops over batches otherwise).  The 12 and 16
// wavefront sizes only where a stage is one block per row (Q4_0's four-block
// stages need more registers than 12 or 16 wavefronts per CU leave).
template <int QT, int EPI>
static hipError_t launch_wide_rows(const GemvArgs& a, int n_seq, int max_blocks, size_t lds, hipStream_t st) {
    const int n_steps = (a.w.N + 1) / 2;
    const int per_cu = (n_steps + device_cus() - 1) / device_cus();
    const int K = a.w.K;
    constexpr bool kWide = ChunkBlocks<QT>::value == 1;
    if (per_cu <= 4) {
        if (K <= 2 * 256 * 4) return launch_one<QT, 64, EPI, 2, 256>(a, n_seq, max_blocks, lds, st);
        if (K <= 4 * 256 * 4) return launch_one<QT, 64, EPI, 4, 256>(a, n_seq, max_blocks, lds, st);
        return launch_one<QT, 64, EPI, 8, 256>(a, n_seq, max_blocks, lds, st);
    }
    if constexpr (kWide) {
        if (per_cu > 8 && per_cu <= 12) {
            if (K <= 2 * 768 * 4) return launch_one<QT, 64, EPI, 2, 768>(a, n_seq, max_blocks, lds, st);
            return launch_one<QT, 64, EPI, 4, 768>(a, n_seq, max_blocks, lds, st);
        }
        if (per_cu > 12 && per_cu <= 16) {
            if (K <= 2 * 1024 * 4) return launch_one<QT, 64, EPI, 2, 1024>(a, n_seq, max_blocks, lds, st);
            return launch_one<QT, 64, EPI, 4, 1024>(a, n_seq, max_blocks, lds, st);
        }
    }
    if (K <= 2 * 512 * 4) return launch_one<QT, 64, EPI, 2>(a, n_seq, max_blocks, lds, st);
    if (K <= 4 * 512 * 4) return launch_one<QT, 64, EPI, 4>(a, n_seq, max_blocks, lds, st);
    return launch_one<QT, 64, EPI, 8>(a, n_seq, max_blocks, lds, st);
}

template <int QT, int EPI>
static hipError_t launch_gemv_lpr(const GemvArgs& a, int lpr, int n_seq, int max_blocks, size_t lds,
                                  hipStream_t st) {
    // XR float4s per thread cover K = XR x 4 x NT columns in one input batch;
    // K < 2048 (the narrower lane groups) always fits the 2-float4 batch
    constexpr int NT = gemv_threads<EPI>();
    switch (lpr) {
        case 64:
            if (EPI != EPI_LOGITS) return launch_wide_rows<QT, EPI>(a, n_seq, max_blocks, lds, st);
            if (a.w.K <= 2 * NT * 4) return launch_one<QT, 64, EPI, 2>(a, n_seq, max_blocks, lds, st);
            if (a.w.K <= 4 * NT * 4) return launch_one<QT, 64, EPI, 4>(a, n_seq, max_blocks, lds, st);
            return launch_one<QT, 64, EPI, 8>(a, n_seq, max_blocks, lds, st);
        case 32: return launch_one<QT, 32, EPI, 2>(a, n_seq, max_blocks, lds, st);
        case 16: return launch_one<QT, 16, EPI, 2>(a, n_seq, max_blocks, lds, st);
        default: return launch_one<QT, 8, EPI, 2>(a, n_seq, max_blocks, lds, st);
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
    if (epi == EPI_RESID && a.norm_g) return hipErrorInvalidValue;   // the residual products take no gain
    const int nb = a.w.K / 32;
    const int lpr = pick_lpr(nb);
    const size_t sums = a.qtype == kQ4_0 || a.qtype == kQ4_K || a.qtype == kQ5_K ? (size_t)nb * 16
                      : (a.qtype == kQ6_K ? (size_t)nb * 32 : 0);
    const size_t lds = (size_t)nb * 96 + (size_t)((nb + 3) & ~3) * 4 + sums;
    switch (a.qtype) {
        case kQ8_0: return launch_gemv_epi<kQ8_0>(a, epi, lpr, n_seq, max_blocks, lds, st);
        case kQ4_0: return launch_gemv_epi<kQ4_0>(a, epi, lpr, n_seq, max_blocks, lds, st);
        case kQ4_K:
            if (a.w.K % 256) return hipErrorInvalidValue;
            return launch_gemv_epi<kQ4_K>(a, epi, lpr, n_seq, max_blocks, lds, st);
        case kQ5_K:
            if (a.w.K % 256) return hipErrorInvalidValue;
            return launch_gemv_epi<kQ5_K>(a, epi, lpr, n_seq, max_blocks, lds, st);
        case kQ6_K:
            if (a.w.K % 256) return hipErrorInvalidValue;
            return launch_gemv_epi<kQ6_K>(a, epi, lpr, n_seq, max_blocks, lds, st);
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------------------
// 2..4 sequences: dequant-GEMV as a dense contraction on the matrix cores
// ---------------------------------------------------------------------------
// v_mfma_i32_16x16x32_i8 contracts a 16 x 32 int8 activation tile with a
// 32-column x 16-row weight tile (one quant block of 16 weight rows, its int8
// quants - or Q4_0 nibbles as unsigned bytes - as they are in HBM).  The
// activations enter as the integer digits of the one-sequence GEMV (per block
// b and sequence s, X = rint(x * 127 * 2^16 / max|x_b|) = D2 2^16 + D1 2^8 +
// D0, signed bytes), and the activation tile's 16 rows are (sequence, digit)
// slots: row 4s + d, slot d = 3 unused.  Operand layout (lane l, group
// g = l/16, index j = l%16):
//   A (digits): row j, block columns 8g..8g+7;
//   B (weights): weight row j of the tile, block columns 8g..8g+7;
//   D: rows 4g..4g+3 (sequence g's three digit sums and the unused slot),
//      column j (weight row j).
// So each lane holds one sequence's digit sums of one weight row and folds
// them itself, block by block: y += d_b * sx_b * (2^16 S2 + 2^8 S1 + S0)
// (Q4_0: S_k minus 8 times the block's digit sum, exactly, in int32 first).
typedef int v4i_t __attribute__((ext_vector_type(4)));

constexpr int kMbWaves = 8;        // wavefronts per workgroup (one workgroup per CU)
constexpr int kMbGroup = 4;        // blocks per pipeline stage (whole fragments of both formats)
constexpr int kMbLdsMaxK = 6144;   // widest input whose digits a workgroup computes into LDS

bool gateup_writes_digits(int64_t ffn) { return ffn > kMbLdsMaxK && ffn % 32 == 0; }

// The digits of 8 consecutive inputs v (a quarter of a 32-column block; the
// block's four quarters sit in lanes 4k..4k+3 of one wavefront): the three
// digit planes packed 8 bytes each, the block's digit sums t[d] (over all 32
// columns) and max|x_b| as the return value.
__device__ __forceinline__ float block_digits(const float (&v)[8], uint2 (&w)[3], int (&t)[3]) {
    float m = 0.f;
    #pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
    // (the block's four lanes are a quad: DPP moves, no LDS round trip)
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, false)));  // quad_perm [1,0,3,2]
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xF, 0xF, false)));  // quad_perm [2,3,0,1]
    const float f = m > 0.f ? 8323072.0f / m : 0.f;         // 127 * 2^16 / max|x_b|
    uint32_t p[3][2] = {{0u, 0u}, {0u, 0u}, {0u, 0u}};
    t[0] = t[1] = t[2] = 0;
    #pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int X = (int)rintf(v[e] * f);
        const int x1 = (X + 128) >> 8, x2 = (x1 + 128) >> 8;
        const int d0 = (int)(int8_t)(X & 255), d1 = (int)(int8_t)(x1 & 255);
        p[0][e >> 2] |= (uint32_t)(d0 & 255) << (8 * (e & 3));
        p[1][e >> 2] |= (uint32_t)(d1 & 255) << (8 * (e & 3));
        p[2][e >> 2] |= (uint32_t)(x2 & 255) << (8 * (e & 3));
        t[0] += d0;
        t[1] += d1;
        t[2] += x2;
    }
    #pragma unroll
    for (int d = 0; d < 3; ++d) {
        t[d] = sum4(t[d]);
        w[d] = make_uint2(p[d][0], p[d][1]);
    }
    return m;
}

// Activation operands (layout also in lm_internal.h, xfrag_bytes), for nb
// blocks: digits uint2 [nb][4 groups g][16 rows 4s+d] (rows 4s+3 unused),
// then the activation scales max|x_b| / (127 * 2^16) fp32 [nb][4 sequences],
// then the digit sums int4 [nb][4 sequences] (S0, S1, S2, 0).
__host__ __device__ constexpr int64_t mb_scales_offset(int64_t nb) { return nb * 512; }
__host__ __device__ constexpr int64_t mb_sums_offset(int64_t nb) { return nb * 512 + nb * 16; }

// Stores one item's digits (sequence s, columns 8c..8c+7) into the operand
// layout at base (LDS or global).
__device__ __forceinline__ void put_digits(uint8_t* base, int nb, int s, int c, const uint2 (&w)[3],
                                           const int (&t)[3], float m) {
    const int b = c >> 2, gq = c & 3;
    uint2* dig = (uint2*)base;
    #pragma unroll
    for (int d = 0; d < 3; ++d) dig[(b * 4 + gq) * 16 + 4 * s + d] = w[d];
    if (gq == 0) {
        ((float*)(base + mb_scales_offset(nb)))[b * 4 + s] = m * (1.0f / 8323072.0f);
        ((int4*)(base + mb_sums_offset(nb)))[b * 4 + s] = make_int4(t[0], t[1], t[2], 0);
    }
}

// Digits of inputs wider than kMbLdsMaxK (the down projection's hidden
// vector, no gain) into a.xfrag, for the four sequence slots (slots past
// n_seq get zeros).  A thread per 8 columns and sequence slot.
__global__ __launch_bounds__(kBlock) void k_xdigits(const float* __restrict__ xin, int x_stride, int K, int n_seq,
                                                   uint8_t* __restrict__ xb) {
    const int s = blockIdx.y, nb = K >> 5;
    const int c = blockIdx.x * kBlock + threadIdx.x;       // 8 columns per thread
    const bool in = c < K / 8;                             // K % 32 == 0: a block's four threads agree
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (in && s < n_seq) {
        const float* x = xin + (int64_t)s * x_stride + 8 * c;
        const float4 v0 = *(const float4*)x, v1 = *(const float4*)(x + 4);
        v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
        v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    }
    uint2 w[3];
    int t[3];
    const float m = block_digits(v, w, t);
    if (in) put_digits(xb, nb, s, c, w, t, m);
}

// Several-sequence GEMV: k_gemv_mb<QT, EPI, TW, XL>.  One workgroup of eight
// wavefronts per CU takes every G-th 16-row tile (G workgroups); its
// wavefronts split K (whole stages of kMbGroup blocks) and take its tiles TW
// at a time: per stage a lane loads, for each of the TW tiles, its weight
// fragments (from the fragment copy: 1 KiB per wavefront, tile and fragment
// group, contiguous) and its row's four block scales, and one activation
// digit fragment per block that serves all TW tiles.  Two stages stay in
// flight; the next round's first stage is requested before the round's
// results are reduced.  A round ends with one LDS reduction over the
// wavefronts, and wavefront t finishes tile t of the round (epilogue lane:
// sequence g, tile row j; even rows take the row pair j, j+1).
// XL: the workgroup computes the digits of every sequence into LDS in its
// prologue (K <= kMbLdsMaxK), while its first stage is in flight, from x
// (times the gain for RMSNorm inputs; the RMS factor of each sequence then
// scales the finished dot products); else they come from a.xfrag (k_xdigits).
template <int QT, int EPI, int TW, bool XL, bool DG>
__global__ __launch_bounds__(64 * kMbWaves) void k_gemv_mb(GemvArgs a) {
    constexpr int NT = 64 * kMbWaves;
    extern __shared__ __align__(16) uint8_t mb_lds[];
    __shared__ float part[2][kMbWaves][TW][64];
    __shared__ float ss_red[kMbWaves][4];
    __shared__ float wv_best[kMbWaves][4];
    __shared__ int wi_best[kMbWaves][4];
    __shared__ int s_last;
    __shared__ float h_blk[DG ? 4 : 1][32];   // DG: a round's SwiGLU outputs, per sequence

    const int K = a.w.K, N = a.w.N, nb = K >> 5;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, j = lane & 15;
    const int n_tiles = (N + 15) >> 4;
    const int G = gridDim.x;
    // this workgroup's tiles: blockIdx.x + G i for i = 0 .. t_end-1, so that at
    // any time the workgroups read neighbouring tiles (one window of the matrix).
    // DG (gate/up whose output feeds a wide-input GEMV): groups of four
    // consecutive tiles instead, group blockIdx.x + G r in round r, so that a
    // round's outputs are one whole 32-column block of h (N % 64 == 0)
    static_assert(!DG || (EPI == EPI_SWIGLU && TW == 4 && XL), "digits from the gate/up rounds");
    const int t_begin = 0;
    const int n_units = DG ? n_tiles >> 2 : n_tiles;
    const int t_end = ((int)blockIdx.x < n_units ? (n_units - 1 - (int)blockIdx.x) / G + 1 : 0) * (DG ? 4 : 1);
    auto tile_at = [&](int i) { return DG ? 4 * ((int)blockIdx.x + G * (i >> 2)) + (i & 3) : (int)blockIdx.x + G * i; };
    const int ng4 = (nb + kMbGroup - 1) / kMbGroup;
    const int k_lo = wave * ng4 / kMbWaves, k_hi = (wave + 1) * ng4 / kMbWaves;
    constexpr int PER = QT == kQ8_0 ? 2 : 4;         // blocks per 16-byte weight fragment
    constexpr int NF = kMbGroup / PER;               // fragments per stage and tile
    const int ngrp = (nb + PER - 1) / PER;

    // LDS: XL: digits, scales, sums (the xfrag layout); else the scales and sums only
    const int64_t tab_off = XL ? mb_scales_offset(nb) : 0;

    constexpr int XS = XL ? 1 : kMbGroup;              // digit operands a stage carries (global digits)
    struct Stage {
        uint4 w[TW][NF];    // weight fragments of this lane's row, per tile
        // scales of the stage's four blocks: TW = 1: this lane's row; else lane l
        // holds those of row l % 16 of tile (l / 16) % TW, each read once per
        // wavefront and handed to the lanes that need them (sc_of)
        uint2 sc;
        uint2 x[XS];        // (digits from a.xfrag) this lane's digit fragment of each block
    };
    // this workgroup's tiles t0.. t0+TW-1 (clamped to its last tile), stage k.
    // Every address is clamped, so a stage's loads are issued unconditionally
    // and the compiler's in-order load counters stay exact.
    auto load = [&](int t0, int k, Stage& st) {
        #pragma unroll
        for (int t = 0; t < TW; ++t) {
            const int tile = tile_at(min(t0 + t, t_end - 1));
            const uint4* qf = (const uint4*)a.w.qf + (int64_t)tile * ngrp * 64 + lane;
            #pragma unroll
            for (int f = 0; f < NF; ++f) st.w[t][f] = ld16_stream(qf + (int64_t)min(k * NF + f, ngrp - 1) * 64);
        }
        {
            const int tile = tile_at(min(t0 + (TW == 1 ? 0 : (lane >> 4) % TW), t_end - 1));
            st.sc = ld8_stream(a.w.sct + (((int64_t)tile * ng4 + k) * 16 + j) * 4);
        }
        if constexpr (!XL) {
            #pragma unroll
            for (int u = 0; u < XS; ++u) {
                const int b = min(k * kMbGroup + u, nb - 1);
                st.x[u] = ((const uint2*)a.xfrag)[(b * 4 + g) * 16 + j];
            }
        }
    };
    float acc[TW];
    auto compute = [&](int k, const Stage& st) {
        // this lane's row's scales for each tile: from lane 16 t + j (TW > 1)
        // (rows 16 t .. 16 t + 15 hold tile t's: broadcast with row swaps)
        uint2 sc_of[TW];
        if constexpr (TW == 1) {
            sc_of[0] = st.sc;
        } else if constexpr (TW == 2) {
            uint32_t bx[2], by[2];
            row_bcast2(st.sc.x, bx);
            row_bcast2(st.sc.y, by);
            sc_of[0] = make_uint2(bx[0], by[0]);
            sc_of[1] = make_uint2(bx[1], by[1]);
        } else {
            uint32_t bx[4], by[4];
            row_bcast4(st.sc.x, bx);
            row_bcast4(st.sc.y, by);
            #pragma unroll
            for (int t = 0; t < TW; ++t) sc_of[t] = make_uint2(bx[t], by[t]);
        }
        #pragma unroll
        for (int u = 0; u < kMbGroup; ++u) {
            const int b = k * kMbGroup + u;
            if (b >= nb) break;
            uint2 xp;
            float sx;
            int4 T = make_int4(0, 0, 0, 0);
            if constexpr (XL) xp = ((const uint2*)mb_lds)[(b * 4 + g) * 16 + j];
            else xp = st.x[u % XS];
            // the scales and sums sit in LDS in both modes (XL: past the digits)
            sx = ((const float*)(mb_lds + tab_off))[b * 4 + g];
            if (QT == kQ4_0) T = ((const int4*)(mb_lds + tab_off + (int64_t)nb * 16))[b * 4 + g];
            const long xv = (long)(((uint64_t)xp.y << 32) | xp.x);
            #pragma unroll
            for (int t = 0; t < TW; ++t) {
                uint2 wa;
                if (QT == kQ8_0) {
                    const uint4 f = st.w[t][u >> 1];
                    wa = (u & 1) ? make_uint2(f.z, f.w) : make_uint2(f.x, f.y);
                } else {
                    // 4 bytes: columns 8g+i in the low nibbles, 8g+4+i in the high ones
                    const uint4 f = st.w[t][0];
                    const uint32_t q = u == 0 ? f.x : u == 1 ? f.y : u == 2 ? f.z : f.w;
                    wa = make_uint2(q & 0x0F0F0F0Fu, (q >> 4) & 0x0F0F0F0Fu);
                }
                const long wv = (long)(((uint64_t)wa.y << 32) | wa.x);
                v4i_t c = {0, 0, 0, 0};
                c = __builtin_amdgcn_mfma_i32_16x16x32_i8(xv, wv, c, 0, 0, 0);
                if (QT == kQ4_0) {                           // nibble n = q + 8
                    c[0] -= 8 * T.x;
                    c[1] -= 8 * T.y;
                    c[2] -= 8 * T.z;
                }
                const uint2 sc = sc_of[t];
                const float d = h2f((uint16_t)(u == 0 ? (sc.x & 0xFFFF) : u == 1 ? (sc.x >> 16)
                                                : u == 2 ? (sc.y & 0xFFFF) : (sc.y >> 16)));
                acc[t] = fmaf(d * sx, combine_digits(c[0], c[1], c[2]), acc[t]);
            }
        }
    };

    // steps i = 0 .. S-1: round i / n_k, stage k_lo + i % n_k.  D stages in
    // flight (deeper measured slower): step i + D - 1 is requested before step i computes (requests
    // past the last step repeat it: clamped, so the load counts the compiler
    // tracks are exact); the first D - 1 go out before the prologue.
    constexpr int D = 2;
    const bool has_k = k_lo < k_hi;
    const int n_rounds = (t_end - t_begin + TW - 1) / TW;
    const int n_k = k_hi - k_lo, S = n_rounds * n_k;
    auto issue = [&](int i, Stage& st) {
        const int ic = min(i, S - 1);
        const int rq = ic / n_k;
        load(t_begin + rq * TW, k_lo + (ic - rq * n_k), st);
    };
    // XL: the prologue's first batch of the input (and the gain) is requested
    // before any weight: the load counters are in order, so the digits can
    // then be computed while the weights are still arriving
    constexpr int MAXI = (kMbLdsMaxK / 8 + NT - 1) / NT;   // prologue batches
    const int cpr = K >> 3;                                   // 8-column items per sequence
    const bool gain = XL && a.norm_g != nullptr;
    float4 xv0[4][2], gv00 = make_float4(1.f, 1.f, 1.f, 1.f), gv01 = gv00;
    if constexpr (XL) {
        const int cc = tid < cpr ? tid : 0;
        if (gain) {
            gv00 = *(const float4*)(a.norm_g + 8 * cc);
            gv01 = *(const float4*)(a.norm_g + 8 * cc + 4);
        }
        #pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float* xs = a.xin + (int64_t)min(s, a.n_seq - 1) * a.x_stride + 8 * cc;
            xv0[s][0] = *(const float4*)xs;
            xv0[s][1] = *(const float4*)(xs + 4);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    Stage st[D];
    if (has_k && t_begin < t_end) {
        #pragma unroll
        for (int p = 0; p < D - 1; ++p) issue(p, st[p]);
    }
    // EPI_RESID: the residual that round 0's finishing lane adds to,
    // requested right behind the first stage (clamped; every workgroup holds
    // at least one tile)
    float2 pre_res = make_float2(0.f, 0.f);
    if (EPI == EPI_RESID) {
        const int tile = tile_at(min(t_begin + min(wave, TW - 1), t_end - 1));
        pre_res = *(const float2*)(a.out + (int64_t)min(g, a.n_seq - 1) * a.out_stride +
                                   min(tile * 16 + (j & ~1), N - 2));
    }

    if constexpr (!XL) {
        // the activation scales and digit sums of every block (nb x 80 bytes,
        // written by k_xdigits) into LDS; the first stage stays in flight
        const int n16 = nb * 5;                             // 16-byte pieces
        const uint4* src = (const uint4*)(a.xfrag + mb_scales_offset(nb));
        for (int i = tid; i < n16; i += NT) ((uint4*)mb_lds)[i] = src[i];
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    // ---- prologue (XL): an item per (8 columns, sequence slot); the four
    // slots of a column group in one thread, so the gain is read once
    float rms = 1.f;            // the RMS factor of this lane's sequence g
    if constexpr (XL) {
        float ssq[4] = {0.f, 0.f, 0.f, 0.f};
        #pragma unroll
        for (int i = 0; i < MAXI; ++i) {
            const int c = tid + i * NT;
            if (i > 0 && c - (tid & 3) >= cpr) break;       // (whole blocks, uniform per block)
            const bool in = c < cpr;
            const int cc = in ? c : 0;
            float4 gv0 = gv00, gv1 = gv01;
            float4 xv[4][2];
            if (i == 0) {
                #pragma unroll
                for (int s = 0; s < 4; ++s) {
                    xv[s][0] = xv0[s][0];
                    xv[s][1] = xv0[s][1];
                }
            } else {
                if (gain) {
                    gv0 = *(const float4*)(a.norm_g + 8 * cc);
                    gv1 = *(const float4*)(a.norm_g + 8 * cc + 4);
                }
                #pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float* xs = a.xin + (int64_t)min(s, a.n_seq - 1) * a.x_stride + 8 * cc;
                    xv[s][0] = *(const float4*)xs;
                    xv[s][1] = *(const float4*)(xs + 4);
                }
            }
            #pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bool live = in && s < a.n_seq;
                float v[8] = {xv[s][0].x, xv[s][0].y, xv[s][0].z, xv[s][0].w,
                              xv[s][1].x, xv[s][1].y, xv[s][1].z, xv[s][1].w};
                if (!live) {
                    #pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = 0.f;
                }
                if (gain) {
                    #pragma unroll
                    for (int e = 0; e < 8; ++e) ssq[s] = fmaf(v[e], v[e], ssq[s]);
                    v[0] *= gv0.x; v[1] *= gv0.y; v[2] *= gv0.z; v[3] *= gv0.w;
                    v[4] *= gv1.x; v[5] *= gv1.y; v[6] *= gv1.z; v[7] *= gv1.w;
                }
                uint2 w[3];
                int t[3];
                const float m = block_digits(v, w, t);
                if (in) put_digits(mb_lds, nb, s, c, w, t, m);
            }
        }
        if (gain) {
            #pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float t = wave_sum(ssq[s]);
                if (lane == 0) ss_red[wave][s] = t;
            }
        }
        // LDS stores visible to the workgroup; the weight loads stay in flight
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (gain) {
            float tot = 0.f;
            #pragma unroll
            for (int w = 0; w < kMbWaves; ++w) tot += ss_red[w][g];
            rms = 1.0f / sqrtf(tot / (float)K + a.eps);
        }
    }

    float best_v = -FLT_MAX;
    int best_i = INT_MAX;
    #pragma unroll
    for (int t = 0; t < TW; ++t) acc[t] = 0.f;
    // end of round rq (tiles t0..t0+TW-1): one LDS reduction over the
    // wavefronts, wavefront t finishes tile t.  Two partial buffers: round
    // rq+1 writes the other one, and round rq+2 this one only after every
    // wavefront has passed round rq+1's barrier, its reduction done.
    auto end_round = [&](int rq, int t0) {
        #pragma unroll
        for (int t = 0; t < TW; ++t) {
            part[rq & 1][wave][t][lane] = acc[t];
            acc[t] = 0.f;
        }
        __syncthreads();
        if (wave < TW && t0 + wave < t_end) {
            const int tile = tile_at(t0 + wave);
            float y = 0.f;
            #pragma unroll
            for (int w = 0; w < kMbWaves; ++w) y += part[rq & 1][w][wave][lane];
            y *= rms;
            // row j + 1 of the same sequence (row_shl:1; lane 15's value is unused)
            const float y1 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(y), 0x101, 0xF, 0xF, false));
            const int s = g, r0 = tile * 16 + j;               // rows r0, r0 + 1 (a RoPE / gate-up pair)
            if (s < a.n_seq && (j & 1) == 0) {
                const float y0 = y;
                if (EPI == EPI_QKV) {
                    const int p = a.pos[s];
                    const int hd = a.head_dim;
                    if (r0 < a.q_rows + a.kv_rows) {
                        const int rr = r0 < a.q_rows ? r0 : r0 - a.q_rows;
                        const int pi = (rr % hd) >> 1;
                        const float cs = a.rope_cos[(int64_t)p * (hd >> 1) + pi];
                        const float sn = a.rope_sin[(int64_t)p * (hd >> 1) + pi];
                        const float z0 = y0 * cs - y1 * sn;
                        const float z1 = y0 * sn + y1 * cs;
                        if (r0 < a.q_rows) {
                            *(float2*)(a.out + (int64_t)s * a.out_stride + r0) = make_float2(z0, z1);
                        } else {
                            __half2* dst = (__half2*)(a.kcache + (int64_t)s * a.kv_seq_stride +
                                                      ((int64_t)(rr / hd) * a.max_ctx + p) * hd + (rr % hd));
                            *dst = __floats2half2_rn(z0, z1);
                        }
                    } else {
                        const int rr = r0 - a.q_rows - a.kv_rows;
                        __half2* dst = (__half2*)(a.vcache + (int64_t)s * a.kv_seq_stride +
                                                  ((int64_t)(rr / hd) * a.max_ctx + p) * hd + (rr % hd));
                        *dst = __floats2half2_rn(y0, y1);
                    }
                } else if (EPI == EPI_RESID) {
                    float* xo = a.out + (int64_t)s * a.out_stride + r0;
                    float2 v = rq == 0 ? pre_res : *(float2*)xo;
                    v.x += y0;
                    v.y += y1;
                    *(float2*)xo = v;
                } else if (EPI == EPI_SWIGLU) {
                    const float sg = y0 / (1.0f + __expf(-y0));
                    a.out[(int64_t)s * a.out_stride + (r0 >> 1)] = sg * y1;
                    if (DG) h_blk[s][8 * wave + (j >> 1)] = sg * y1;
                } else {  // EPI_LOGITS: the vocabulary may end inside a tile or a pair
                    if (r0 < N) {
                        if (a.out) a.out[(int64_t)s * a.out_stride + r0] = y0;
                        better(best_v, best_i, y0, r0);
                    }
                    if (r0 + 1 < N) {
                        if (a.out) a.out[(int64_t)s * a.out_stride + r0 + 1] = y1;
                        better(best_v, best_i, y1, r0 + 1);
                    }
                }
            }
        }
        if constexpr (DG) {
            // the round's 32 outputs of every sequence are h's block
            // t0 / 4 + ... (its group): its digits for the wide GEMV that reads
            // h next, as k_xdigits would compute them from the same fp32
            // values (sequence slots past n_seq get zeros).  Round rq + 1
            // writes h_blk only after its own first barrier, which the
            // digit lanes reach after these reads.
            __syncthreads();
            if (tid < 16) {
                const int sq = tid >> 2, qd = tid & 3;        // sequence slot, 8-column quarter
                float v[8];
                #pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = sq < a.n_seq ? h_blk[sq][8 * qd + e] : 0.f;
                uint2 w[3];
                int tq[3];
                const float m = block_digits(v, w, tq);
                const int blk = tile_at(t0) >> 2;
                put_digits(a.xfrag, N >> 6, sq, 4 * blk + qd, w, tq, m);
            }
        }
    };

    if (has_k) {
        auto run = [&](int i, const Stage& sg) {
            const int rq = i / n_k, k = k_lo + (i - rq * n_k);
            compute(k, sg);
            if (k == k_hi - 1) end_round(rq, t_begin + rq * TW);
        };
        // whole groups of D steps (no exit inside a group, so each stage
        // keeps its registers), then the last < D steps, already requested
        int i = 0;
        for (; i + D <= S; i += D) {
            #pragma unroll
            for (int u = 0; u < D; ++u) {
                issue(i + u + D - 1, st[(u + D - 1) % D]);
                run(i + u, st[u]);
            }
        }
        #pragma unroll
        for (int u = 0; u < D - 1; ++u)
            if (i + u < S) run(i + u, st[u]);
    } else {
        for (int rq = 0; rq < n_rounds; ++rq) end_round(rq, t_begin + rq * TW);
    }

    if (EPI == EPI_LOGITS) {
        // this workgroup's best row per sequence: over the tile rows (lanes j
        // of group g), then the wavefronts; handed to the last workgroup as the
        // attention chunks hand over their states (lm_device.h)
        group_argmax<16>(best_v, best_i);
        if (j == 0) {
            wv_best[wave][g] = best_v;
            wi_best[wave][g] = best_i;
        }
        __syncthreads();
        if (tid < a.n_seq) {
            float bv = wv_best[0][tid];
            int bi = wi_best[0][tid];
            for (int w = 1; w < kMbWaves; ++w) better(bv, bi, wv_best[w][tid], wi_best[w][tid]);
            st_dev(&a.part_val[(int64_t)tid * G + blockIdx.x], bv);
            st_dev(&a.part_idx[(int64_t)tid * G + blockIdx.x], bi);
        }
        drain_vm();
        __syncthreads();
        if (tid == 0) s_last = count_arrive(&a.counter[0], G);
        __syncthreads();
        if (s_last) {
            for (int s = 0; s < a.n_seq; ++s) {
                float bv = -FLT_MAX;
                int bi = INT_MAX;
                for (int i = tid; i < G; i += NT)
                    better(bv, bi, ld_dev(&a.part_val[(int64_t)s * G + i]), ld_dev(&a.part_idx[(int64_t)s * G + i]));
                group_argmax<64>(bv, bi);
                if (lane == 0) {
                    wv_best[wave][s] = bv;
                    wi_best[wave][s] = bi;
                }
            }
            __syncthreads();
            if (tid == 0) {
                for (int s = 0; s < a.n_seq; ++s) {
                    float bv = wv_best[0][s];
                    int bi = wi_best[0][s];
                    for (int w = 1; w < kMbWaves; ++w) better(bv, bi, wv_best[w][s], wi_best[w][s]);
                    a.argmax_out[s] = bi;
                    if (a.pos_inc) a.pos_inc[s] += 1;
                }
            }
        }
    }
}

template <int QT, int EPI, int TW, bool XL, bool DG = false>
static hipError_t launch_mb(const GemvArgs& a, int max_blocks, hipStream_t st) {
    const int n_tiles = (a.w.N + 15) / 16, nb = a.w.K / 32;
    if (!XL && !a.xfrag_ready) {
        hipLaunchKernelGGL(k_xdigits, dim3((a.w.K / 8 + kBlock - 1) / kBlock, 4), dim3(kBlock), 0, st, a.xin,
                           a.x_stride, a.w.K, a.n_seq, a.xfrag);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // XL: digits, scales, sums; else scales and sums
    const size_t lds = XL ? (size_t)mb_sums_offset(nb) + (size_t)nb * 64 : (size_t)nb * 80;
    const int grid = std::max(1, std::min({DG ? n_tiles / 4 : n_tiles, device_cus(), max_blocks}));
    hipLaunchKernelGGL((k_gemv_mb<QT, EPI, TW, XL, DG>), dim3(grid), dim3(64 * kMbWaves), lds, st, a);
    return hipGetLastError();
}

// TW from the tiles per workgroup (one workgroup per CU): up to four tiles
// per round share each digit fragment
template <int QT, int EPI>
static hipError_t launch_mb_shape(const GemvArgs& a, int max_blocks, hipStream_t st) {
    const int n_tiles = (a.w.N + 15) / 16;
    const int per = (n_tiles + device_cus() - 1) / device_cus();
    if (a.w.K > kMbLdsMaxK) {
        if (a.norm_g) return hipErrorInvalidValue;           // (the wide inputs take no gain)
        if (per >= 4) return launch_mb<QT, EPI, 4, false>(a, max_blocks, st);
        if (per >= 2) return launch_mb<QT, EPI, 2, false>(a, max_blocks, st);
        return launch_mb<QT, EPI, 1, false>(a, max_blocks, st);
    }
    // gate/up whose output h is wider than the prologue digits: its rounds
    // write h's digits for the down projection (k_xdigits not launched)
    if constexpr (EPI == EPI_SWIGLU)
        if (gateup_writes_digits(a.w.N / 2)) return launch_mb<QT, EPI, 4, true, true>(a, max_blocks, st);
    if (per >= 4) return launch_mb<QT, EPI, 4, true>(a, max_blocks, st);
    if (per >= 2) return launch_mb<QT, EPI, 2, true>(a, max_blocks, st);
    return launch_mb<QT, EPI, 1, true>(a, max_blocks, st);
}

hipError_t launch_gemv_batched(const GemvArgs& a0, int epi, int n_seq, int max_blocks, hipStream_t st) {
    if (n_seq < 1 || n_seq > 4 || !a0.w.sct || !a0.w.qf || !a0.xfrag) return hipErrorInvalidValue;
    if (a0.w.K % 32) return hipErrorInvalidValue;
    GemvArgs a = a0;
    a.n_seq = n_seq;
    if (a.qtype == kQ8_0) {
        switch (epi) {
            case EPI_QKV: return launch_mb_shape<kQ8_0, EPI_QKV>(a, max_blocks, st);
            case EPI_RESID: return launch_mb_shape<kQ8_0, EPI_RESID>(a, max_blocks, st);
            case EPI_SWIGLU: return launch_mb_shape<kQ8_0, EPI_SWIGLU>(a, max_blocks, st);
            default: return launch_mb_shape<kQ8_0, EPI_LOGITS>(a, max_blocks, st);
        }
    }
    if (a.qtype != kQ4_0) return hipErrorInvalidValue;
    switch (epi) {
        case EPI_QKV: return launch_mb_shape<kQ4_0, EPI_QKV>(a, max_blocks, st);
        case EPI_RESID: return launch_mb_shape<kQ4_0, EPI_RESID>(a, max_blocks, st);
        case EPI_SWIGLU: return launch_mb_shape<kQ4_0, EPI_SWIGLU>(a, max_blocks, st);
        default: return launch_mb_shape<kQ4_0, EPI_LOGITS>(a, max_blocks, st);
    }
}

// ---------------------------------------------------------------------------
// GQA decode attention with causal softmax, split over context
// ---------------------------------------------------------------------------
// One workgroup of four wavefronts per (span of TP 64-position tiles, KV
// head, sequence); wavefront w takes keys 16w..16w+15 of every tile of the
// span and runs its own online softmax over them, so a tile needs no
// exchange between wavefronts.  The group's G query heads (at most
// kMaxGroup, padded to 16) go through v_mfma_f32_16x16x16f16 twice per tile:
//   scores, transposed: S^T[key][head] = sum_d K[key][d] q[head][d], with K
//     as the first operand straight from the loaded registers (lane: key l%16,
//     dimension pieces 8(4u + l/16) .. +7 of its row, 16-byte loads) and q as
//     the second in the same dimension order; q enters as two fp16 terms,
//     hi = fp16(q), lo = fp16(q - hi) (q to about 2^-22 relative; K is fp16
//     already), fp32 accumulation.  A lane's four results are keys
//     4(l/16)..+3 of head l%16: the layout of the probabilities as the first
//     operand of the next product, so they never leave the lane;
//   o[head][d] += sum_key p[head][key] V[key][d]: the wavefront's 16 V rows
//     pass through its own LDS rows (loaded as whole 128-byte lines, read
//     back by columns; rows past the context written as zeros, so a
//     probability of 0 never meets a stale cache value), p as fp16 hi + lo.
// At the end of the span the four wavefronts' states (maximum, sum, o) are
// combined in LDS.  A context that fits one span writes o directly;
// otherwise each span publishes its softmax state (m, l, o) with device-
// coherent stores, and the last span of the (sequence, KV head) to finish
// merges all of them (merge_chunk_states) within the same launch.
constexpr int kMaxGroup = 8;   // query heads per KV head
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));

template <int HD>
__global__ __launch_bounds__(kBlock) void k_attn(AttnArgs a) {
    static_assert(kBlock == 256 && kAttnChunk == 64, "four wavefronts, sixteen keys each");
    constexpr int CH = kAttnChunk;
    constexpr int KP = HD + 8;                  // padded V row (halves): conflict-free column reads
    constexpr int KL = HD / 32;                 // 16-byte pieces of a K (and of a V) row per lane
    constexpr int KS = HD / 16;                 // 16-dimension steps of the score product
    constexpr int DT = HD / 16;                 // 16-column tiles of o
    __shared__ __align__(16) __half Vw[4][16][KP];   // each wavefront's own V rows
    __shared__ __align__(16) float Mw[4][16];
    __shared__ float Lw[4][16];
    __shared__ int s_last;
    // after the tiles: the wavefronts' o, then the merge scratch
    float* xs = reinterpret_cast<float*>(&Vw[0][0][0]);
    static_assert(sizeof(float) * 4 * kMaxGroup * HD <= sizeof(Vw), "o exchange fits in Vw");
    static_assert(sizeof(float) * 6 * kBlock <= sizeof(Vw), "merge scratch fits in Vw");

    const int chunk = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;   // operand row / column index, lane group
    const int G = a.nq / a.nkv;
    const int64_t stride = HD + 2;              // partial record (even: 8-byte aligned pairs)

    // ---- the first tile's loads first (rows clamped to the cache; masked below)
    const __half* Kg = a.kcache + (int64_t)s * a.kv_seq_stride + (int64_t)g * a.max_ctx * HD;
    const __half* Vg = a.vcache + (int64_t)s * a.kv_seq_stride + (int64_t)g * a.max_ctx * HD;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // (native vectors: kept in registers)
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const int TP = a.tiles;                     // tiles of this workgroup's span
    const int t_first = chunk * TP;
    // tile t's K and V pieces of this lane.  K: key 64t + 16 wave + lr,
    // pieces 4u + lq (the matrix-op operand layout).  V, which passes through
    // LDS: whole 128-byte lines per load instruction (eight rows: row
    // vrow_of(u), dimensions 64 (u % (HD / 64)) + 8 (lane % 8) .. +7), with the
    // non-temporal hint (the hint helps only whole-line requests; K keeps
    // plain loads)
    auto vrow_of = [&](int u) { return 8 * (u / (HD / 64)) + (lane >> 3); };
    auto vcol_of = [&](int u) { return 64 * (u % (HD / 64)) + 8 * (lane & 7); };
    auto load = [&](int t, u32x4 (&kr)[KL], u32x4 (&vr)[KL]) {
        const int64_t row = min(t * CH + 16 * wave + lr, a.max_ctx - 1);
        #pragma unroll
        for (int u = 0; u < KL; ++u) {
            kr[u] = *(const u32x4*)(Kg + row * HD + 8 * (4 * u + lq));
            const int64_t vrow = min(t * CH + 16 * wave + vrow_of(u), a.max_ctx - 1);
            vr[u] = __builtin_nontemporal_load((const u32x4*)(Vg + vrow * HD + vcol_of(u)));
        }
    };
    // this lane's q operands: head lr (zero past G), at step k the dimensions
    // 32(k/2) + 8lq + 4(k%2) .. +3 (the order of its K pieces).  Requested
    // first (needed first: the load counters are in order), then the first
    // tile's K and V, all before any wait: one round trip.
    const float* qg = a.q + (int64_t)s * a.nq * HD + (int64_t)g * G * HD + (int64_t)min(lr, G - 1) * HD;
    float4 qv[KS];
    #pragma unroll
    for (int k = 0; k < KS; ++k) qv[k] = *(const float4*)(qg + 32 * (k >> 1) + 8 * lq + 4 * (k & 1));
    u32x4 ka[KL], va[KL], kb[KL], vb[KL];
    load(t_first, ka, va);
    __builtin_amdgcn_sched_barrier(0);   // (the scheduler would otherwise hold V back behind the waits)
    const int n_ctx = a.pos[s] + 1;                       // keys 0..pos inclusive
    const int n_tiles = (n_ctx + CH - 1) / CH;
    const int n_act = (n_tiles + TP - 1) / TP;            // spans holding keys
    if (chunk >= n_act) return;                           // span past the causal horizon

    h4_t qh[KS], ql[KS];
    #pragma unroll
    for (int k = 0; k < KS; ++k) {
        const float v[4] = {qv[k].x, qv[k].y, qv[k].z, qv[k].w};
        #pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x = lr < G ? v[e] : 0.f;
            const _Float16 hi = (_Float16)x;
            qh[k][e] = hi;
            ql[k][e] = (_Float16)(x - (float)hi);
        }
    }
    // running state of this wavefront: maximum and sum of head lr (the same
    // in the four lane groups), o[dt][i]: head 4lq + i, dimension 16dt + lr
    float M = -FLT_MAX, L = 0.f;
    f4_t o[DT];
    #pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f4_t{0.f, 0.f, 0.f, 0.f};

    // one tile (a tile past the context has no valid key and changes nothing)
    auto step = [&](int tile, const u32x4 (&kr)[KL], const u32x4 (&vr)[KL]) {
        // scores of keys 4lq + i (of this wavefront's 16), head lr
        f4_t sh = {0.f, 0.f, 0.f, 0.f}, sl = {0.f, 0.f, 0.f, 0.f};
        #pragma unroll
        for (int k = 0; k < KS; ++k) {
            const u32x4 pc = kr[k >> 1];
            const h4_t kk = __builtin_bit_cast(h4_t, (k & 1) ? u32x2{pc.z, pc.w} : u32x2{pc.x, pc.y});
            sh = __builtin_amdgcn_mfma_f32_16x16x16f16(kk, qh[k], sh, 0, 0, 0);
            sl = __builtin_amdgcn_mfma_f32_16x16x16f16(kk, ql[k], sl, 0, 0, 0);
        }
        // this wavefront's V rows into its LDS rows (past the context: zeros)
        #pragma unroll
        for (int u = 0; u < KL; ++u) {
            const bool vlive = tile * CH + 16 * wave + vrow_of(u) < n_ctx;
            *(u32x4*)&Vw[wave][vrow_of(u)][vcol_of(u)] = vlive ? vr[u] : u32x4{0u, 0u, 0u, 0u};
        }
        // online softmax of head lr over this wavefront's keys
        const int key0 = tile * CH + 16 * wave + 4 * lq;
        float sv[4], mt = -FLT_MAX;
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            sv[i] = key0 + i < n_ctx ? (sh[i] + sl[i]) * a.scale : -FLT_MAX;
            mt = fmaxf(mt, sv[i]);
        }
        mt = max_xor32(max_xor16(mt));
        const float mn = fmaxf(M, mt);
        const float r = __expf(M - mn);                   // 0 on the first live tile
        M = mn;
        h4_t pa, pb;
        float ps = 0.f;
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = key0 + i < n_ctx ? __expf(sv[i] - mn) : 0.f;
            const _Float16 ph = (_Float16)p;
            pa[i] = ph;
            pb[i] = (_Float16)(p - (float)ph);
            ps += p;
        }
        ps = sum_xor32(sum_xor16(ps));
        L = fmaf(L, r, ps);
        // the rescale of o's heads 4lq + i: r of head h sits in lane h (heads
        // past kMaxGroup are padding: lanes lq >= 2 take any finite factor)
        float rh[8];
        #pragma unroll
        for (int h = 0; h < 8; ++h) rh[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), h));
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ri = lq == 0 ? rh[i] : rh[4 + i];
            #pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt][i] *= ri;
        }
        // the V rows written above, read by columns (this wavefront's own
        // rows: its LDS operations complete in order once counted)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        #pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            h4_t vv;
            #pragma unroll
            for (int e = 0; e < 4; ++e) vv[e] = *(const _Float16*)&Vw[wave][4 * lq + e][16 * dt + lr];
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vv, o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(pb, vv, o[dt], 0, 0, 0);
        }
        // the next tile's V stores come after these reads
        asm volatile("" ::: "memory");
    };
    // the next tile's loads are requested before this one computes (the
    // scheduling barriers keep them there).  Whole pairs of tiles first (no
    // exit inside a pair, so each buffer keeps its registers), then the last
    // one or two.
    int ti = 0;
    for (; ti + 2 < TP; ti += 2) {
        load(t_first + ti + 1, kb, vb);
        __builtin_amdgcn_sched_barrier(0);
        step(t_first + ti, ka, va);
        load(t_first + ti + 2, ka, va);
        __builtin_amdgcn_sched_barrier(0);
        step(t_first + ti + 1, kb, vb);
    }
    const bool two = ti + 1 < TP;
    if (two) load(t_first + ti + 1, kb, vb);
    __builtin_amdgcn_sched_barrier(0);
    step(t_first + ti, ka, va);
    if (two) step(t_first + ti + 1, kb, vb);

    // ---- the four wavefronts' states: the span's maximum per head, each
    // wavefront's o scaled to it, summed in LDS
    if (lq == 0) {
        Mw[wave][lr] = M;
        Lw[wave][lr] = L;
    }
    __syncthreads();
    {
        // heads 4lq .. 4lq + 3 of this lane's o: the four wavefronts' maxima
        float4 mw[4];
        #pragma unroll
        for (int w = 0; w < 4; ++w) mw[w] = *(const float4*)&Mw[w][4 * lq];
        const float4 own = *(const float4*)&Mw[wave][4 * lq];
        const float mo[4] = {own.x, own.y, own.z, own.w};
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float m0 = i == 0 ? mw[0].x : i == 1 ? mw[0].y : i == 2 ? mw[0].z : mw[0].w;
            const float m1 = i == 0 ? mw[1].x : i == 1 ? mw[1].y : i == 2 ? mw[1].z : mw[1].w;
            const float m2 = i == 0 ? mw[2].x : i == 1 ? mw[2].y : i == 2 ? mw[2].z : mw[2].w;
            const float m3 = i == 0 ? mw[3].x : i == 1 ? mw[3].y : i == 2 ? mw[3].z : mw[3].w;
            const float f = __expf(mo[i] - fmaxf(fmaxf(m0, m1), fmaxf(m2, m3)));
            if (4 * lq + i < G) {
                #pragma unroll
                for (int dt = 0; dt < DT; ++dt) xs[(wave * G + 4 * lq + i) * HD + 16 * dt + lr] = o[dt][i] * f;
            }
        }
    }
    __syncthreads();

    // a thread per (head, 4 dimensions): the sum over the wavefronts
    float* part_s = a.part + (int64_t)s * a.nq * a.max_chunks * stride;
    float* out_s = a.out + (int64_t)s * a.nq * HD + (int64_t)g * G * HD;
    for (int idx = tid; idx < G * HD / 4; idx += kBlock) {
        const int h = idx / (HD / 4), d = (idx % (HD / 4)) * 4;
        const float mt = fmaxf(fmaxf(Mw[0][h], Mw[1][h]), fmaxf(Mw[2][h], Mw[3][h]));
        float lt = 0.f;
        float4 ot = make_float4(0.f, 0.f, 0.f, 0.f);
        #pragma unroll
        for (int w = 0; w < 4; ++w) {
            lt = fmaf(Lw[w][h], __expf(Mw[w][h] - mt), lt);
            const float4 v = *(const float4*)&xs[(w * G + h) * HD + d];
            ot.x += v.x;
            ot.y += v.y;
            ot.z += v.z;
            ot.w += v.w;
        }
        if (n_act == 1) {
            const float inv = 1.f / lt;
            *(float4*)(out_s + h * HD + d) = make_float4(ot.x * inv, ot.y * inv, ot.z * inv, ot.w * inv);
        } else {
            float* ph = part_s + ((int64_t)(g * G + h) * a.max_chunks + chunk) * stride;
            st_dev2(ph + d, ot.x, ot.y);
            st_dev2(ph + d + 2, ot.z, ot.w);
            if (d == 0) st_dev2(ph + HD, mt, lt);
        }
    }
    if (n_act == 1) return;

    // ---- the last span of this (sequence, KV head) merges every span.  The
    // partials are device-coherent stores; each wavefront waits for its own
    // to complete before the count is taken.
    drain_vm();
    __syncthreads();
    if (tid == 0)
        s_last = chunk_arrive(a.counter + (int64_t)(s * a.nkv + g) * attn_cnt_lines(a.max_chunks) * kCntStride,
                              chunk, n_act);
    __syncthreads();
    if (!s_last) return;

    const float* part_g = part_s + (int64_t)g * G * a.max_chunks * stride;
    merge_chunk_states<HD>(
        G, n_act, [&](int j) { return part_g + (int64_t)j * a.max_chunks * stride; },
        [](const float* p) { return ld_dev2(p); },
        [&](int i, float4 v) { *(float4*)(out_s + i) = v; },
        reinterpret_cast<float (*)[6]>(xs));
}

// Tiles per attention workgroup: as few as keep the whole grid resident at
// once (the workgroups one CU holds, from the kernel's registers and LDS,
// times the CUs), so no workgroup waits for another to finish, and longer
// spans leave fewer partial states to merge; but at least three once the
// context holds 20 chunks (measured on the 8B and 1B shapes, one and four
// sequences: 3-tile spans beat 1 and 2 there, up to 16.5 -> 11.6 us at 4000
// positions, while 512 positions keep 1).
int attn_tiles(int n_seq, int nkv, int max_chunks, int hd) {
    static int per_cu[2] = {0, 0};
    int& pc = per_cu[hd == 128 ? 1 : 0];
    if (!pc) {
        const void* f = hd == 128 ? (const void*)k_attn<128> : (const void*)k_attn<64>;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&pc, f, kBlock, 0) != hipSuccess || pc < 1) pc = 1;
    }
    const int64_t tiles = (int64_t)n_seq * nkv * max_chunks, slots = (int64_t)pc * device_cus();
    const int64_t resident = std::max<int64_t>(1, (tiles + slots - 1) / slots);
    return (int)std::max<int64_t>(resident, max_chunks >= 20 ? 3 : 1);
}

hipError_t launch_attention(const AttnArgs& a, int n_seq, hipStream_t st) {
    if (a.tiles < 1) return hipErrorInvalidValue;
    if (a.hd != 128 && a.hd != 64) return hipErrorInvalidValue;
    if (a.grid_chunks < 1 || a.grid_chunks > a.max_chunks) return hipErrorInvalidValue;
    if (a.nq % a.nkv || a.nq / a.nkv > kMaxGroup) return hipErrorInvalidValue;
    dim3 grid((a.grid_chunks + a.tiles - 1) / a.tiles, a.nkv, n_seq);
    if (a.hd == 128) hipLaunchKernelGGL((k_attn<128>), grid, dim3(kBlock), 0, st, a);
    else hipLaunchKernelGGL((k_attn<64>), grid, dim3(kBlock), 0, st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// inspection kernels
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void k_dequant(QMat w, int qtype, int row0, float* __restrict__ out) {
    const int r = row0 + blockIdx.x;
    const int K = w.K, nb = K >> 5;
    const int64_t rowq = qmat_qbytes(qtype, 1, K);
    const int64_t srow = qmat_srow(qtype, K) / 2;     // 16-bit words
    const uint8_t* q = w.q + (int64_t)r * rowq;
    const uint16_t* sc = w.sc + (int64_t)r * srow;
    // Q8_0 / Q4_0: with paired scales, this row's at every other word of its row pair's
    const uint16_t* sp = kScPairs ? w.sc + (int64_t)(r & ~1) * srow + (r & 1) : sc;
    const int sstep = kScPairs ? 2 : 1;
    for (int c = threadIdx.x; c < K; c += kBlock) {
        const int b = c >> 5, e = c & 31;
        float v;
        if (qtype == kQ8_0) {
            const float d = h2f(sp[sstep * b]);
            const int8_t qi = (int8_t)(e < 16 ? q[b * 16 + e] : q[(int64_t)nb * 16 + b * 16 + (e - 16)]);
            v = d * (float)qi;
        } else {
            const uint8_t byte = q[b * 16 + (e & 15)];
            const int nib = e < 16 ? (byte & 0xF) : (byte >> 4);
            if (qtype == kQ4_0) {
                v = (float)(nib - 8) * h2f(sp[sstep * b]);
            } else if (qtype == kQ4_K || qtype == kQ5_K) {
                float ds, dm;
                q4k_scale_min(*(const int4*)(sc + (b >> 3) * 8), b & 7, ds, dm);
                int q5 = nib;
                if (qtype == kQ5_K) {
                    const int ii = e & 15;
                    const uint8_t hb = q[(int64_t)nb * 16 + b * 4 + (ii & 3)];
                    q5 |= ((hb >> ((ii >> 2) + (e < 16 ? 0 : 4))) & 1) << 4;
                }
                v = fmaf(ds, (float)q5, -dm);                   // one rounding of the exact value
            } else {  // Q6_K
                const int ii = e & 15;
                const uint8_t hb = q[(int64_t)nb * 16 + b * 8 + 4 * (e >> 4) + (ii & 3)];
                const int q6 = nib | (((hb >> (2 * (ii >> 2))) & 3) << 4);
                const int8_t s6 = (int8_t)(e < 16 ? (sc[b] & 255) : (sc[b] >> 8));
                v = h2f(sc[nb + (b >> 3)]) * (float)s6 * (float)(q6 - 32);   // exact in fp32
            }
        }
        out[(int64_t)blockIdx.x * K + c] = v;
    }
}

hipError_t launch_dequant(const QMat& w, int qtype, int row0, int n_rows, float* out, hipStream_t st) {
    hipLaunchKernelGGL(k_dequant, dim3(n_rows), dim3(kBlock), 0, st, w, qtype, row0, out);
    return hipGetLastError();
}

// Layer similarity (the C/CUDA Llama engine page, sections 3.5 and 4.5: the
// cosine similarity of a layer's input and output hidden vectors, calibrated
// ahead of time): for each sequence, cos = a.b / (|a| |b|) in fp64 (0 when
// either vector is zero); acc[0] += the cosines, acc[1] += the sequences.
// One workgroup, sequences in order: the sums are deterministic.
__global__ __launch_bounds__(kBlock) void k_layer_cos(const float* __restrict__ xin, const float* __restrict__ x,
                                                     int H, int n_seq, double* __restrict__ acc) {
    __shared__ double red[3][kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    double tot = 0.0;
    for (int s = 0; s < n_seq; ++s) {
        double ab = 0.0, aa = 0.0, bb = 0.0;
        for (int i = tid; i < H; i += kBlock) {
            const double av = xin[(int64_t)s * H + i], bv = x[(int64_t)s * H + i];
            ab = fma(av, bv, ab);
            aa = fma(av, av, aa);
            bb = fma(bv, bv, bb);
        }
        for (int off = 32; off > 0; off >>= 1) {
            ab += __shfl_xor(ab, off, 64);
            aa += __shfl_xor(aa, off, 64);
            bb += __shfl_xor(bb, off, 64);
        }
        if (lane == 0) { red[0][wave] = ab; red[1][wave] = aa; red[2][wave] = bb; }
        __syncthreads();
        if (tid == 0) {
            double sab = 0.0, saa = 0.0, sbb = 0.0;
            for (int w = 0; w < kWaves; ++w) { sab += red[0][w]; saa += red[1][w]; sbb += red[2][w]; }
            tot += (saa == 0.0 || sbb == 0.0) ? 0.0 : sab / (sqrt(saa) * sqrt(sbb));
        }
        __syncthreads();
    }
    if (tid == 0) {
        acc[0] += tot;
        acc[1] += (double)n_seq;
    }
}

hipError_t launch_layer_cos(const float* xin, const float* x, int H, int n_seq, double* acc, hipStream_t st) {
    hipLaunchKernelGGL(k_layer_cos, dim3(1), dim3(kBlock), 0, st, xin, x, H, n_seq, acc);
    return hipGetLastError();
}

__global__ __launch_bounds__(kBlock) void k_read_bw(const uint4* __restrict__ buf, int64_t n16,
                                                   float* __restrict__ sink) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n16; i += stride) {
        const uint4 v = ld16_stream(buf + i);     // the loads the GEMVs stream their weights with
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    acc = (uint32_t)wave_sum((float)(acc & 0xFFFF));
    if (threadIdx.x == 0) sink[blockIdx.x] = (float)acc;
}

hipError_t launch_read_bw(const void* buf, int64_t n_bytes, float* sink, hipStream_t st) {
    hipLaunchKernelGGL(k_read_bw, dim3(2048), dim3(kBlock), 0, st, (const uint4*)buf, n_bytes / 16, sink);
    return hipGetLastError();
}

__global__ __launch_bounds__(kBlock) void k_zero(uint32_t* __restrict__ p, int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n4; i += stride) p[i] = 0u;
}

hipError_t launch_zero(void* p, int64_t n_bytes, hipStream_t st) {
    if (n_bytes < 0 || n_bytes % 4 || ((uintptr_t)p & 3)) return hipErrorInvalidValue;
    if (n_bytes == 0) return hipSuccess;
    const int64_t n4 = n_bytes / 4;
    const int grid = (int)std::min<int64_t>(1024, (n4 + kBlock - 1) / kBlock);
    hipLaunchKernelGGL(k_zero, dim3(grid), dim3(kBlock), 0, st, (uint32_t*)p, n4);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// scratch of the allocation-free step
// ---------------------------------------------------------------------------
// A fixed array in the code object: every device the library runs on holds
// its own copy, from when the code object is loaded there until the process
// ends, and every call on that device shares it.  In host code its name is
// not a device address; the address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(int device, uint8_t** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static uint8_t* addr[kMaxDevices] = {};
    if (device < 0 || device >= kMaxDevices || !ptr) return hipErrorInvalidValue;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (cur != device) {
            const hipError_t r = hipSetDevice(cur);
            if (e == hipSuccess) e = r;
        }
        if (e != hipSuccess) return e;
        if (!a) return hipErrorInvalidSymbol;
        addr[device] = (uint8_t*)a;
    }
    *ptr = addr[device];
    return hipSuccess;
}

}  // namespace lmk
