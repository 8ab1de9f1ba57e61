// lm_flow.hip - every layer of a batch-1 decode step in one launch, with the
// workgroups ordered by dependency (gfx950).
//
// The operators are those of the per-operator kernels (C/CUDA Llama engine
// page, rskf.cn/news/15116, section 4.4): per layer RMSNorm + QKV GEMV + RoPE
// + KV append, GQA attention with the causal softmax, Wo + residual,
// RMSNorm + gate/up GEMV + SwiGLU, down + residual.
//
// MI355X design.  Launch boundaries cost a fixed ~2 us each on this chip, and
// a GEMV kernel's weight stream only starts after its launch, so a step of
// 160 short kernels spends a large share of its time with HBM idle.  Here the
// grid is the concatenation of every phase's workgroups (layer-major, phase
// order QKV, attention, Wo, gate/up, down).  A workgroup
//   1. requests the first weights it multiplies (or, for attention, the K/V
//      rows of earlier positions) - these depend on nothing of this step;
//   2. waits until every workgroup of the phase before it has finished (a
//      per-phase device counter);
//   3. reads its input vector, runs its part of the phase and
//   4. signals: waits for its own stores, then adds one to its phase counter.
// Workgroups are dispatched in index order on each XCD, and a workgroup only
// waits on lower-indexed ones, so the lowest unfinished workgroup is always
// resident and never waiting: the chain cannot deadlock.  While one phase
// drains, the next phase's workgroups already occupy the freed slots with
// their weight requests in flight, so the HBM stream does not stop at phase
// boundaries.
//
// Activations that cross workgroups inside the launch (x, q, o, h, the new
// K/V row, attention partials) move through device-coherent relaxed atomic
// loads and stores (the L2 of one XCD is not coherent with the others).
// Everything written before the launch (weights, older K/V rows, the
// position) is read with ordinary loads.  Every wait is bounded: a timeout
// sets an error flag, and a workgroup that sees it skips its work but still
// signals, so the grid always drains.
#include "lm_flow.h"
#include "lm_device.h"

#include <float.h>
#include <limits.h>

#include <algorithm>

namespace lmk {
namespace {

constexpr int kSpin = 1 << 22;    // polls (about 1 us each) before a wait gives up
constexpr int kCh = kAttnChunk;   // positions per attention workgroup
constexpr int kHd = 128;          // head dimension of the supported shapes
constexpr int kMaxG = 8;          // query heads per KV head
constexpr int kFlowWgPerCu = 2;   // resident workgroups per CU
constexpr int kLdsPerCu = 163840;

#define LMF_G __attribute__((address_space(1)))
template <class T> __device__ __forceinline__ LMF_G T* gpf(T* p) { return (LMF_G T*)p; }

__device__ __forceinline__ float ldc(const float* p) {
    return __hip_atomic_load(gpf(const_cast<float*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(float* p, float v) {
    __hip_atomic_store(gpf(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ldc32(const uint32_t* p) {
    return __hip_atomic_load(gpf(const_cast<uint32_t*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc32(uint32_t* p, uint32_t v) {
    __hip_atomic_store(gpf(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ldc64(const void* p) {
    return __hip_atomic_load(gpf((uint64_t*)const_cast<void*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc2(float* p, float x, float y) {
    const uint64_t v = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
    __hip_atomic_store(gpf((uint64_t*)p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t addc32(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(gpf(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int addci(int* p, int v) {
    return __hip_atomic_fetch_add(gpf(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stci(int* p, int v) {
    __hip_atomic_store(gpf(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 ldc4(const float* p) {
    const uint64_t lo = ldc64(p), hi = ldc64(p + 2);
    return make_float4(__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                       __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32)));
}
__device__ __forceinline__ uint4 ldc16(const void* p) {
    const uint64_t lo = ldc64(p), hi = ldc64((const uint8_t*)p + 8);
    return make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
}
// this wavefront's outstanding memory operations have completed (gfx9 vmcnt(0))
__device__ __forceinline__ void drain_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until every one of the `n_wg` workgroups of phase `ph` has finished
// in this launch (ph < 0: no wait): until all of the phase's partial counters
// are complete.  One lane polls; the others wait at the
// barrier.  The launch number (completed launches, `*ep` on lane 0, with bit
// 32 set once known) is read
// here together with the first poll, after the caller's weight requests:
// reading it at the start would hold those requests for its round trip.
// Returns false when the step has been abandoned (timeout here or elsewhere).
__shared__ uint64_t s_twait;      // debug trace: when the wait passed

__device__ bool wait_phase(const FlowArgs& a, int ph, int n_wg, uint64_t* ep) {
    __shared__ int s_ok;
    if (threadIdx.x == 0) {
        int ok = 1;
        if (ph >= 0) {
            const uint32_t* top = a.done + ((int64_t)ph * (kFlowSub + 1) + kFlowSub) * kFlowLine;
            const uint32_t e = ldc32(a.epoch);
            uint32_t v = ldc32(top);
            const uint32_t target = (e + 1u) * (uint32_t)min(n_wg, kFlowSub);
            *ep = (1ull << 32) | e;     // known
            for (int n = 0; (int32_t)(v - target) < 0; ++n) {
                if ((n & 63) == 63) {
                    if (ldc32(a.err) != 0) { ok = 0; break; }
                    if (n > kSpin) { stc32(a.err, 1); ok = 0; break; }
                }
                __builtin_amdgcn_s_sleep(1);
                v = ldc32(top);
            }
        }
        __atomic_store_n(&s_ok, ok, __ATOMIC_RELAXED);
        if (a.trace) s_twait = __builtin_amdgcn_s_memrealtime();
    }
    // a bare barrier: the flag is LDS, so only LDS completion is needed; a
    // __syncthreads here would also wait for the weight requests in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    return __atomic_load_n(&s_ok, __ATOMIC_RELAXED) != 0;
}

// Weight blocks one lane loads per pipeline stage (per row of its row pair).
template <int QT> struct FChunk {
    static constexpr int CB = QT == kQ8_0 ? LMK_CB_Q8 : LMK_CB_Q4;
    int4 a0[CB], a1[CB];
    int4 b0[QT == kQ8_0 ? CB : 1], b1[QT == kQ8_0 ? CB : 1];
    uint16_t d0[CB], d1[CB];
};

// ---------------------------------------------------------------------------
// GEMV phases: the integer-digit dequant-GEMV of the per-operator kernel with
// all 64 lanes of a wavefront on one row pair, its input read device-coherently
// after the wait, and device-coherent epilogue traffic.
//   QKV   : RMSNorm(x) -> q (RoPE) | K row (RoPE) | V row of this position
//   RESID : x += W in          (Wo: in = o; down: in = h)
//   SWIGLU: RMSNorm(x) -> h = silu(gate) * up, rows interleaved (gate i, up i)
// ---------------------------------------------------------------------------
template <int QT, int EPI, int XR>
__device__ void flow_gemv(const FlowArgs& a, int l, int wg, int n_wg, const FlowMat& fm, const float* xin,
                          const float* gain, float* out, int ph_wait, int n_prev, uint64_t* ep, uint8_t* smem,
                          float* red) {
    constexpr int LPR = 64;
    constexpr int CB = FChunk<QT>::CB;
    constexpr bool kGain = EPI != EPI_RESID;
    const uint8_t* blob = a.blobs + (int64_t)l * a.blob_stride;
    const uint8_t* wq = blob + fm.q_off;
    const uint16_t* wsc = (const uint16_t*)(blob + fm.sc_off);
    const int K = fm.K, N = fm.N, nb = K >> 5;
    int8_t* xq = (int8_t*)smem;                       // [nb][3][32] digit planes
    float* xsc = (float*)(xq + nb * 96);              // [nb] block scales
    int4* dsum = (int4*)(xsc + ((nb + 3) & ~3));      // [nb] digit sums (Q4_0)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane;
    const int64_t rowq = QT == kQ8_0 ? (int64_t)K : (int64_t)(K >> 1);

    // row pairs: wavefront w of workgroup b takes pairs w*G + b, then + 4G, ...
    // (G workgroups), so every workgroup gets the same number of pairs within
    // one; where a workgroup runs does not then decide how long its CU works
    const int n_steps = (N + 1) / 2;
    const int step0 = wave * n_wg + wg, sstride = n_wg * kWaves;
    const int my_steps = step0 < n_steps ? (n_steps - 1 - step0) / sstride + 1 : 0;
    const int bpl = (nb + LPR - 1) / LPR;
    const int cps = (bpl + CB - 1) / CB;
    const int n_chunks = my_steps * cps;

    auto load = [&](int c, FChunk<QT>& w) {
        const int i = c / cps, k = c - i * cps;
        const int r0 = min((step0 + i * sstride) * 2, N - 2);
        const uint8_t* q0 = wq + (int64_t)r0 * rowq;
        const uint8_t* q1 = q0 + rowq;
        const uint16_t* s0 = wsc + (int64_t)r0 * nb;
        #pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int b = li + LPR * (k * CB + u);
            const uint32_t bc = (uint32_t)min(b, nb - 1);
            w.a0[u] = ld16_stream(q0 + bc * 16u);
            w.a1[u] = ld16_stream(q1 + bc * 16u);
            if (QT == kQ8_0) {
                w.b0[u] = ld16_stream(q0 + (uint32_t)nb * 16u + bc * 16u);
                w.b1[u] = ld16_stream(q1 + (uint32_t)nb * 16u + bc * 16u);
            }
            w.d0[u] = s0[bc];
            w.d1[u] = s0[(uint32_t)nb + bc];
        }
    };

    float acc0 = 0.f, acc1 = 0.f;
    auto compute = [&](int c, const FChunk<QT>& w) {
        const int k = c % cps;
        #pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int braw = li + LPR * (k * CB + u);
            const int b = min(braw, nb - 1);
            const float d0 = braw < nb ? h2f(w.d0[u]) : 0.f;
            const float d1 = braw < nb ? h2f(w.d1[u]) : 0.f;
            const int4* D = (const int4*)(xq + b * 96);
            const float sx = xsc[b];
            if (QT == kQ8_0) {
                acc0 = fmaf(d0 * sx, dot_q8(w.a0[u], w.b0[u], D), acc0);
                acc1 = fmaf(d1 * sx, dot_q8(w.a1[u], w.b1[u], D), acc1);
            } else {
                const int4 T = dsum[b];
                acc0 = fmaf(d0 * sx, dot_q4(w.a0[u], D, T), acc0);
                acc1 = fmaf(d1 * sx, dot_q4(w.a1[u], D, T), acc1);
            }
        }
    };

    // ---- 1. the first two weight chunks: independent of this step's activations
    FChunk<QT> wa, wb;
    load(0, wa);
    load(1, wb);

    // ---- 2. wait for the producing phase
    if (!wait_phase(a, ph_wait, n_prev, ep)) return;

    // ---- 3. input (device-coherent) -> integer digits in LDS, RMSNorm folded in
    float ss = 0.f;
    for (int base = 0; base < K; base += XR * kBlock * 4) {
        float4 xr[XR], gr[kGain ? XR : 1];
        #pragma unroll
        for (int u = 0; u < XR; ++u) {
            const int i = min(base + (tid + u * kBlock) * 4, K - 4);
            xr[u] = ldc4(xin + i);
            if (kGain) gr[u] = *(const float4*)(gain + i);
        }
        #pragma unroll
        for (int u = 0; u < XR; ++u) {
            const int i = base + (tid + u * kBlock) * 4;
            float4 v = xr[u];
            if (kGain) {
                if (i < K) {
                    ss = fmaf(v.x, v.x, ss);
                    ss = fmaf(v.y, v.y, ss);
                    ss = fmaf(v.z, v.z, ss);
                    ss = fmaf(v.w, v.w, ss);
                }
                const float4 gv = gr[kGain ? u : 0];
                v.x *= gv.x;
                v.y *= gv.y;
                v.z *= gv.z;
                v.w *= gv.w;
            }
            stage_digits(v, i, K, xq, xsc, dsum, QT == kQ4_0);
        }
    }
    float rscale = 1.f;
    if (kGain) rscale = 1.0f / sqrtf(block_sum(ss, red) / (float)K + a.eps);
    __syncthreads();

    // ---- epilogue inputs of the first row pair (RoPE tables / residual)
    const int pos = EPI == EPI_QKV ? a.pos[0] : 0;
    const int hd = a.hd, q_rows = a.nq * a.hd, kv_rows = a.nkv * a.hd;
    float pre_cs = 1.f, pre_sn = 0.f, pre_x0 = 0.f, pre_x1 = 0.f;
    {
        const int r0 = min(step0 * 2, N - 2);
        if (EPI == EPI_QKV) {
            const int rc = min(r0, q_rows + kv_rows - 2);
            const int rr = rc < q_rows ? rc : rc - q_rows;
            const int pi = (rr % hd) >> 1;
            pre_cs = a.rope_cos[(int64_t)pos * (hd >> 1) + pi];
            pre_sn = a.rope_sin[(int64_t)pos * (hd >> 1) + pi];
        } else if (EPI == EPI_RESID) {
            pre_x0 = ldc(out + r0);
            pre_x1 = ldc(out + r0 + 1);
        }
    }
    __half* kc = a.kcache + (int64_t)l * a.kv_layer;
    __half* vc = a.vcache + (int64_t)l * a.kv_layer;

    auto finish = [&](int c) {
        if (c % cps != cps - 1) return;
        const int i = c / cps;
        const int r0 = (step0 + i * sstride) * 2;
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
            if (r0 < q_rows + kv_rows) {
                const int rr = r0 < q_rows ? r0 : r0 - q_rows;
                const int pi = (rr % hd) >> 1;
                const float cs = i == 0 ? pre_cs : a.rope_cos[(int64_t)pos * (hd >> 1) + pi];
                const float sn = i == 0 ? pre_sn : a.rope_sin[(int64_t)pos * (hd >> 1) + pi];
                const float z0 = y0 * cs - y1 * sn;
                const float z1 = y0 * sn + y1 * cs;
                if (r0 < q_rows) {
                    stc(a.q + r0, z0);
                    stc(a.q + r0 + 1, z1);
                } else {
                    const int g = rr / hd;
                    const __half2 hv = __floats2half2_rn(z0, z1);
                    stc32((uint32_t*)(kc + ((int64_t)g * a.max_ctx + pos) * hd + (rr % hd)),
                          *(const uint32_t*)&hv);
                }
            } else {
                const int rr = r0 - q_rows - kv_rows;
                const int g = rr / hd;
                const __half2 hv = __floats2half2_rn(y0, y1);
                stc32((uint32_t*)(vc + ((int64_t)g * a.max_ctx + pos) * hd + (rr % hd)), *(const uint32_t*)&hv);
            }
        } else if (EPI == EPI_RESID) {
            const float x0 = i == 0 ? pre_x0 : ldc(out + r0);
            const float x1 = i == 0 ? pre_x1 : ldc(out + r0 + 1);
            stc(out + r0, x0 + y0);
            stc(out + r0 + 1, x1 + y1);
        } else {   // EPI_SWIGLU: row 2i = gate i, row 2i+1 = up i
            const float sg = y0 / (1.0f + __expf(-y0));
            stc(out + (r0 >> 1), sg * y1);
        }
    };

    // ---- 4. the weight pipeline (two chunks in flight), as in the per-operator kernel
    int c = 0;
    for (; c + 3 < n_chunks; c += 2) {
        compute(c, wa);
        load(c + 2, wa);
        finish(c);
        compute(c + 1, wb);
        load(c + 3, wb);
        finish(c + 1);
    }
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
}

// ---------------------------------------------------------------------------
// attention phase: one workgroup per (64-position chunk, KV head); the last
// chunk of a KV head to finish merges the partial softmax states (as in the
// per-operator kernel).  The K/V rows of earlier positions are requested
// before the wait; the new row (this step's) is re-read device-coherently.
// ---------------------------------------------------------------------------
template <int HD>
__device__ void flow_attn(const FlowArgs& a, int l, int wg, int ph_wait, int n_prev, uint64_t* ep, uint8_t* smem) {
    constexpr int CH = kCh;
    constexpr int KP = HD + 8;                   // padded K row (halves)
    constexpr int PCS = CH * HD / 8 / kBlock;    // 16-byte pieces per thread per tile
    static_assert(sizeof(float) * kWaves * kMaxG * HD <= sizeof(__half) * CH * KP, "Os fits in Ks");
    __half (*Ks)[KP] = (__half (*)[KP])smem;
    __half (*Vs)[HD] = (__half (*)[HD])(smem + sizeof(__half) * CH * KP);
    float (*Qs)[HD] = (float (*)[HD])(smem + sizeof(__half) * CH * (KP + HD));
    float (*Ps)[CH] = (float (*)[CH])((uint8_t*)Qs + sizeof(float) * kMaxG * HD);
    float* Ms = (float*)((uint8_t*)Ps + sizeof(float) * kMaxG * CH);
    float* Ls = Ms + kMaxG;
    __shared__ int s_last;
    float (*Os)[kMaxG * HD] = (float (*)[kMaxG * HD])smem;   // reuses Ks after the scores

    const int chunk = wg % a.max_chunks, g = wg / a.max_chunks;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = a.nq / a.nkv;
    const int t0 = chunk * CH;
    const int p = a.pos[0];
    const int n_ctx = p + 1;                       // keys 0..p inclusive
    const int n_act = (n_ctx + CH - 1) / CH;
    if (chunk >= n_act) return;                    // past the causal horizon (uniform)
    const int nt = min(CH, n_ctx - t0);
    const int64_t stride = HD + 2;

    // ---- 1. K/V rows of this chunk (rows clamped to the cache; masked below)
    const __half* Kg = a.kcache + (int64_t)l * a.kv_layer + (int64_t)g * a.max_ctx * HD;
    const __half* Vg = a.vcache + (int64_t)l * a.kv_layer + (int64_t)g * a.max_ctx * HD;
    uint4 kr[PCS], vr[PCS];
    #pragma unroll
    for (int u = 0; u < PCS; ++u) {
        const int c = tid + u * kBlock;
        const int t = min(t0 + c / (HD / 8), a.max_ctx - 1), d8 = (c % (HD / 8)) * 8;
        kr[u] = *(const uint4*)(Kg + (int64_t)t * HD + d8);
        vr[u] = *(const uint4*)(Vg + (int64_t)t * HD + d8);
    }

    // ---- 2. wait for the QKV phase
    if (!wait_phase(a, ph_wait, n_prev, ep)) return;

    // ---- 3. the new row and the rotated queries (device-coherent)
    #pragma unroll
    for (int u = 0; u < PCS; ++u) {
        const int c = tid + u * kBlock;
        const int t = t0 + c / (HD / 8), d8 = (c % (HD / 8)) * 8;
        if (t == p) {
            kr[u] = ldc16(Kg + (int64_t)t * HD + d8);
            vr[u] = ldc16(Vg + (int64_t)t * HD + d8);
        }
    }
    const float* qg = a.q + (int64_t)g * G * HD;
    constexpr int kQ = (kMaxG * HD / 4 + kBlock - 1) / kBlock;
    float4 qv[kQ];
    #pragma unroll
    for (int u = 0; u < kQ; ++u) {
        const int i = min((tid + u * kBlock) * 4, G * HD - 4);
        qv[u] = ldc4(qg + i);
    }
    #pragma unroll
    for (int u = 0; u < PCS; ++u) {
        const int c = tid + u * kBlock;
        const int t = c / (HD / 8), d8 = (c % (HD / 8)) * 8;
        *(uint4*)&Ks[t][d8] = kr[u];
        *(uint4*)&Vs[t][d8] = vr[u];
    }
    #pragma unroll
    for (int u = 0; u < kQ; ++u) {
        const int i = (tid + u * kBlock) * 4;
        if (i < G * HD) *(float4*)&Qs[i / HD][i % HD] = qv[u];
    }
    __syncthreads();

    // ---- scores: a wavefront per query head, a lane per key
    for (int j = wave; j < G; j += kWaves) {
        float sc = -FLT_MAX;
        if (lane < nt) {
            float acc0 = 0.f, acc1 = 0.f;
            #pragma unroll
            for (int d = 0; d < HD; d += 8) {
                const uint4 kk = *(const uint4*)&Ks[lane][d];
                const float4 q0 = *(const float4*)&Qs[j][d];
                const float4 q1 = *(const float4*)&Qs[j][d + 4];
                const float2 k01 = __half22float2(*(const __half2*)&kk.x);
                const float2 k23 = __half22float2(*(const __half2*)&kk.y);
                const float2 k45 = __half22float2(*(const __half2*)&kk.z);
                const float2 k67 = __half22float2(*(const __half2*)&kk.w);
                acc0 = fmaf(q0.x, k01.x, acc0);
                acc1 = fmaf(q0.y, k01.y, acc1);
                acc0 = fmaf(q0.z, k23.x, acc0);
                acc1 = fmaf(q0.w, k23.y, acc1);
                acc0 = fmaf(q1.x, k45.x, acc0);
                acc1 = fmaf(q1.y, k45.y, acc1);
                acc0 = fmaf(q1.z, k67.x, acc0);
                acc1 = fmaf(q1.w, k67.y, acc1);
            }
            sc = (acc0 + acc1) * a.scale;
        }
        const float m = wave_max(sc);
        const float pr = lane < nt ? __expf(sc - m) : 0.f;
        const float ls = wave_sum(pr);
        Ps[j][lane] = pr;
        if (lane == 0) { Ms[j] = m; Ls[j] = ls; }
    }
    __syncthreads();

    // ---- o = sum_t p_t v_t: thread (head j, 8 dims, quarter w of the keys)
    constexpr int D8 = HD / 8;
    for (int idx = tid; idx < G * D8 * kWaves; idx += kBlock) {
        const int w = idx / (G * D8), r = idx % (G * D8);
        const int j = r / D8, d8 = (r % D8) * 8;
        float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const int tb = w * (CH / kWaves), te = min(tb + CH / kWaves, nt);
        for (int t = tb; t < te; ++t) {
            const float pt = Ps[j][t];
            const uint4 vv = *(const uint4*)&Vs[t][d8];
            const float2 v01 = __half22float2(*(const __half2*)&vv.x);
            const float2 v23 = __half22float2(*(const __half2*)&vv.y);
            const float2 v45 = __half22float2(*(const __half2*)&vv.z);
            const float2 v67 = __half22float2(*(const __half2*)&vv.w);
            o[0] = fmaf(pt, v01.x, o[0]);
            o[1] = fmaf(pt, v01.y, o[1]);
            o[2] = fmaf(pt, v23.x, o[2]);
            o[3] = fmaf(pt, v23.y, o[3]);
            o[4] = fmaf(pt, v45.x, o[4]);
            o[5] = fmaf(pt, v45.y, o[5]);
            o[6] = fmaf(pt, v67.x, o[6]);
            o[7] = fmaf(pt, v67.y, o[7]);
        }
        float* dst = &Os[w][j * HD + d8];
        *(float4*)dst = make_float4(o[0], o[1], o[2], o[3]);
        *(float4*)(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
    __syncthreads();

    float* out = a.o + (int64_t)g * G * HD;
    if (n_act == 1) {
        for (int i = tid; i < G * HD; i += kBlock) {
            float v = Os[0][i];
            #pragma unroll
            for (int w = 1; w < kWaves; ++w) v += Os[w][i];
            stc(out + i, v / Ls[i / HD]);
        }
        return;
    }
    for (int i = 2 * tid; i < G * HD; i += 2 * kBlock) {
        float v0 = Os[0][i], v1 = Os[0][i + 1];
        #pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            v0 += Os[w][i];
            v1 += Os[w][i + 1];
        }
        const int j = i / HD, d = i % HD;
        float* ph = a.attn_part + ((int64_t)(g * G + j) * a.max_chunks + chunk) * stride;
        stc2(ph + d, v0, v1);
        if (d == 0) stc2(ph + HD, Ms[j], Ls[j]);
    }
    // the last chunk of this KV head merges every chunk
    drain_vm();
    __syncthreads();
    if (tid == 0)
        s_last = chunk_arrive(a.attn_cnt + (int64_t)g * attn_cnt_lines(a.max_chunks) * kCntStride, chunk, n_act);
    __syncthreads();
    if (!s_last) return;
    const float* part_g = a.attn_part + (int64_t)g * G * a.max_chunks * stride;
    merge_chunk_states<HD>(
        G, n_act, [&](int j) { return part_g + (int64_t)j * a.max_chunks * stride; },
        [](const float* p) {
            const uint64_t v = ldc64(p);
            return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
        },
        [&](int i, float4 v) {
            stc2(out + i, v.x, v.y);
            stc2(out + i + 2, v.z, v.w);
        },
        (float (*)[6])smem);
}

// one phase of layer l for workgroup `wg` of the phase's `n_wg`
template <int QT, int XRH, int XRF>
__device__ void flow_phase(const FlowArgs& a, int l, int op, int wg, int n_wg, int ph_prev, int n_prev, uint64_t* ep,
                           uint8_t* smem, float* red) {
    const float* g_attn = a.norms + (int64_t)l * 2 * a.H;
    switch (op) {
        case 0:
            flow_gemv<QT, EPI_QKV, XRH>(a, l, wg, n_wg, a.mat[0], a.x, g_attn, a.q, ph_prev, n_prev, ep, smem, red);
            break;
        case 1:
            // items (chunk, KV head); more than one per workgroup when there are
            // fewer workgroups than items
            for (int it = wg; it < a.nkv * a.max_chunks; it += n_wg) {
                if (it != wg) __syncthreads();      // the previous item's LDS reads are done
                flow_attn<kHd>(a, l, it, ph_prev, n_prev, ep, smem);
            }
            break;
        case 2:
            flow_gemv<QT, EPI_RESID, XRH>(a, l, wg, n_wg, a.mat[1], a.o, nullptr, a.x, ph_prev, n_prev, ep, smem, red);
            break;
        case 3:
            flow_gemv<QT, EPI_SWIGLU, XRH>(a, l, wg, n_wg, a.mat[2], a.x, g_attn + a.H, a.h, ph_prev, n_prev, ep, smem,
                                          red);
            break;
        default:
            flow_gemv<QT, EPI_RESID, XRF>(a, l, wg, n_wg, a.mat[3], a.h, nullptr, a.x, ph_prev, n_prev, ep, smem, red);
            break;
    }
}

// Signal (lane 0): this workgroup has finished phase `ph`, whose `n`
// workgroups have indices first .. first+n-1 (`self` is this one's).
// Two-level count: the workgroup's partial counter (index mod kFlowSub), and,
// from the workgroup completing that partial, the phase's count of complete
// partials (what the next phase polls).  Spreading the atomics over kFlowSub
// lines keeps them from queueing on one address.
__device__ void flow_count(const FlowArgs& a, int ph, int first, int n, int self, uint64_t* ep) {
    if (!(*ep >> 32)) *ep = (1ull << 32) | ldc32(a.epoch);     // a workgroup that did not wait
    const uint32_t e = (uint32_t)*ep;
    const int sub = self % kFlowSub;
    // workgroups of this phase whose index is sub modulo kFlowSub
    const int lo = (first + kFlowSub - 1 - sub) / kFlowSub, hi = (first + n + kFlowSub - 1 - sub) / kFlowSub;
    const uint32_t n_sub = (uint32_t)(hi - lo);
    uint32_t* pc = a.done + ((int64_t)ph * (kFlowSub + 1) + sub) * kFlowLine;
    uint32_t* top = a.done + ((int64_t)ph * (kFlowSub + 1) + kFlowSub) * kFlowLine;
    if (addc32(pc, 1u) + 1u == (e + 1u) * n_sub) {
        const uint32_t done = addc32(top, 1u) + 1u;
        if (ph == a.L * kFlowOps - 1 && done == (e + 1u) * (uint32_t)min(n, kFlowSub))
            stc32(a.epoch, e + 1u);   // the whole grid has finished
    }
}

__device__ void flow_trace(const FlowArgs& a, int64_t row, uint64_t t_start) {
    uint64_t* t = a.trace + row * kFlowTraceWords;
    t[0] = t_start;
    t[1] = s_twait;
    t[2] = __builtin_amdgcn_s_memrealtime();
    // hardware ids: HW_ID (CU, SE, ...) and XCC_ID
    t[3] = ((uint64_t)__builtin_amdgcn_s_getreg((4 << 0) | (0 << 6) | (31 << 11)) << 32) |
           (uint64_t)__builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (15 << 11));
}

// Dataflow launch: one workgroup per (phase, share), layer-major.
template <int QT, int XRH, int XRF>
__global__ __launch_bounds__(kBlock) void k_flow(FlowArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ float red[kWaves];
    const int per_layer = a.wg_off[kFlowOps];
    const int l = blockIdx.x / per_layer;
    const int r = blockIdx.x - l * per_layer;
    int op = 0;
    while (op + 1 < kFlowOps && r >= a.wg_off[op + 1]) ++op;
    const int wg = r - a.wg_off[op];
    const int ph = l * kFlowOps + op;
    uint64_t ep = 0;    // launches completed before this one (lane 0, read in the wait; bit 32: known)
    const uint64_t t_start = a.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    if (a.trace && threadIdx.x == 0) s_twait = 0;
    flow_phase<QT, XRH, XRF>(a, l, op, wg, a.wg[op], ph - 1, a.wg[(op + kFlowOps - 1) % kFlowOps], &ep, smem, red);
    // ---- signal: this workgroup's stores have completed, then count it
    drain_vm();
    __syncthreads();
    if (threadIdx.x == 0) {
        if (a.trace) flow_trace(a, blockIdx.x, t_start);
        flow_count(a, ph, blockIdx.x - wg, a.wg[op], blockIdx.x, &ep);
    }
}

// Resident launch: every workgroup (two per CU, all resident together) takes
// its share of every phase in turn.  After signalling a phase it goes straight
// on to request its first weights of the next, so those requests overlap the
// rest of the grid finishing the phase.  Needs every workgroup resident: a
// wait that cannot be met times out into the error flag.
template <int QT, int XRH, int XRF>
__global__ __launch_bounds__(kBlock, kFlowWgPerCu) void k_flow_res(FlowArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ float red[kWaves];
    const int G = gridDim.x;
    uint64_t ep = 0;
    for (int ph = 0; ph < a.L * kFlowOps; ++ph) {
        const int l = ph / kFlowOps, op = ph - l * kFlowOps;
        const uint64_t t_start = a.trace ? __builtin_amdgcn_s_memrealtime() : 0;
        if (a.trace && threadIdx.x == 0) s_twait = 0;
        flow_phase<QT, XRH, XRF>(a, l, op, blockIdx.x, G, ph - 1, G, &ep, smem, red);
        drain_vm();
        __syncthreads();
        if (threadIdx.x == 0) {
            if (a.trace) flow_trace(a, (int64_t)ph * G + blockIdx.x, t_start);
            flow_count(a, ph, 0, G, blockIdx.x, &ep);
        }
    }
}

int xr_for(int K) { return K <= 4 * kBlock * 4 ? 4 : K <= 8 * kBlock * 4 ? 8 : 16; }

template <int QT, int XRH, int XRF>
hipError_t launch_t(const FlowArgs& a, int lds, hipStream_t st) {
    // the resident kernel keeps two workgroups per CU within 256 registers a
    // lane: its down-projection input comes in batches of at most 8 float4s
    constexpr int XRF_RES = XRF < 8 ? XRF : 8;
    const void* fn = a.resident ? (const void*)k_flow_res<QT, XRH, XRF_RES> : (const void*)k_flow<QT, XRH, XRF>;
    if (lds > 65536) {
        // wide FFN inputs (the 70B shape's 28672 columns): dynamic LDS past the
        // default limit, up to the CU's 160 KB
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
    }
    if (a.resident) {
        // every workgroup must be resident at once: refuse a plan the occupancy does not allow
        int per_cu = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_flow_res<QT, XRH, XRF_RES>, kBlock, lds);
        if (e != hipSuccess) return e;
        int dev = 0, cus = 0;
        if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
        if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        if ((int64_t)per_cu * cus < a.wg[0]) return hipErrorCooperativeLaunchTooLarge;
        hipLaunchKernelGGL((k_flow_res<QT, XRH, XRF_RES>), dim3(a.wg[0]), dim3(kBlock), lds, st, a);
    } else {
        hipLaunchKernelGGL((k_flow<QT, XRH, XRF>), dim3(a.L * a.wg_off[kFlowOps]), dim3(kBlock), lds, st, a);
    }
    return hipGetLastError();
}

template <int QT, int XRH, int XRF>
int per_cu_t(bool resident, int lds) {
    constexpr int XRF_RES = XRF < 8 ? XRF : 8;
    int n = 0;
    const hipError_t e = resident
        ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_flow_res<QT, XRH, XRF_RES>, kBlock, lds)
        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_flow<QT, XRH, XRF>, kBlock, lds);
    return e == hipSuccess ? n : 0;
}

template <int QT>
int per_cu_q(const FlowArgs& a, int lds) {
    const int xh = xr_for(a.H), xf = xr_for(a.F);
    if (xh == 4 && xf == 4) return per_cu_t<QT, 4, 4>(a.resident, lds);
    if (xh == 4 && xf == 8) return per_cu_t<QT, 4, 8>(a.resident, lds);
    if (xh == 4) return per_cu_t<QT, 4, 16>(a.resident, lds);
    if (xf == 8) return per_cu_t<QT, 8, 8>(a.resident, lds);
    return per_cu_t<QT, 8, 16>(a.resident, lds);
}

template <int QT>
hipError_t launch_q(const FlowArgs& a, int lds, hipStream_t st) {
    const int xh = xr_for(a.H), xf = xr_for(a.F);
    if (xh == 4 && xf == 4) return launch_t<QT, 4, 4>(a, lds, st);
    if (xh == 4 && xf == 8) return launch_t<QT, 4, 8>(a, lds, st);
    if (xh == 4) return launch_t<QT, 4, 16>(a, lds, st);
    if (xf == 8) return launch_t<QT, 8, 8>(a, lds, st);
    return launch_t<QT, 8, 16>(a, lds, st);
}

int attn_lds_bytes(int hd) {
    return (int)(sizeof(__half) * kCh * (hd + 8 + hd) + sizeof(float) * kMaxG * hd + sizeof(float) * kMaxG * kCh +
                 sizeof(float) * 2 * kMaxG + 16);
}
int gemv_lds_bytes(int qtype, int K) {
    const int nb = K / 32;
    return nb * 96 + ((nb + 3) & ~3) * 4 + (qtype == kQ4_0 ? nb * 16 : 0);
}

}  // namespace

bool flow_supported(int qtype, int H, int F, int hd, int nq, int nkv) {
    if (qtype != kQ8_0 && qtype != kQ4_0) return false;
    if (hd != kHd || nkv <= 0 || nq % nkv != 0 || nq / nkv > kMaxG) return false;
    if (H < 2048 || F < 2048 || H % 32 != 0 || F % 32 != 0) return false;
    return flow_lds_bytes(qtype, H, F, hd) + 1024 <= kLdsPerCu;   // + the static LDS
}

int flow_lds_bytes(int qtype, int H, int F, int hd) {
    const int g = std::max(gemv_lds_bytes(qtype, H), gemv_lds_bytes(qtype, F));
    // at least a third of the CU's LDS: at most kFlowWgPerCu workgroups per CU
    const int floor_bytes = kLdsPerCu / (kFlowWgPerCu + 1) + 16;
    return (std::max({g, attn_lds_bytes(hd), floor_bytes}) + 15) / 16 * 16;
}

void flow_plan(FlowArgs& a, int qtype, int n_cus) {
    // Two workgroups per CU (the LDS request allows no more) and, for every
    // GEMV phase, exactly as many workgroups as there are slots: the slots a
    // phase frees are then all taken by the next phase, which therefore lands
    // two workgroups on every CU, however unevenly the previous one drained.
    // Rows are dealt so that every workgroup of a phase has the same work.
    auto pairs_wg = [](int N) { return ((N + 1) / 2 + kWaves - 1) / kWaves; };
    const int lds = flow_lds_bytes(qtype, a.H, a.F, a.hd);
    const int occ = qtype == kQ8_0 ? per_cu_q<kQ8_0>(a, lds) : per_cu_q<kQ4_0>(a, lds);
    const int slots = std::max(1, std::min(kFlowWgPerCu, occ)) * n_cus;
    if (a.resident) {
        // the resident launch: every phase has all of them
        for (int i = 0; i < kFlowOps; ++i) a.wg[i] = slots;
        a.wg_off[0] = 0;
        for (int i = 0; i < kFlowOps; ++i) a.wg_off[i + 1] = a.wg_off[i] + a.wg[i];
        return;
    }
    a.wg[0] = std::min(pairs_wg(a.mat[0].N), slots);
    a.wg[1] = a.nkv * a.max_chunks;
    a.wg[2] = std::min(pairs_wg(a.mat[1].N), slots);
    a.wg[3] = std::min(pairs_wg(a.mat[2].N), slots);
    a.wg[4] = std::min(pairs_wg(a.mat[3].N), slots);
    a.wg_off[0] = 0;
    for (int i = 0; i < kFlowOps; ++i) a.wg_off[i + 1] = a.wg_off[i] + a.wg[i];
}

hipError_t launch_flow(const FlowArgs& a, int qtype, hipStream_t st) {
    if (!flow_supported(qtype, a.H, a.F, a.hd, a.nq, a.nkv)) return hipErrorInvalidValue;
    for (int i = 0; i < kFlowOps; ++i)
        if (a.wg[i] < 1) return hipErrorInvalidValue;
    const int lds = flow_lds_bytes(qtype, a.H, a.F, a.hd);
    if (qtype == kQ8_0) return launch_q<kQ8_0>(a, lds, st);
    return launch_q<kQ4_0>(a, lds, st);
}

}  // namespace lmk
