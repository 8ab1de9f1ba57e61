// lm_device.h - device helpers shared by the decode kernels (gfx950): the
// integer-digit dot products of the dequant-GEMV, activation staging,
// wavefront reductions, the lowest-index argmax rule and the merge of
// split-context attention states.
#pragma once

#include "lm_internal.h"

#include <float.h>
#include <limits.h>

// Tuning knobs (compile-time): blocks per lane per pipeline stage, and
// whether weight loads carry the non-temporal hint.
#ifndef LMK_CB_Q8
#define LMK_CB_Q8 1
#endif
#ifndef LMK_CB_Q4
#define LMK_CB_Q4 4
#endif
#ifndef LMK_CB_QK
#define LMK_CB_QK 1     // the K formats (more registers per block: headers / high bits)
#endif

namespace lmk {

constexpr int kBlock = 256;   // threads per workgroup (4 wavefronts)
constexpr int kWaves = kBlock / 64;
// The one-sequence GEMV runs one 8-wavefront workgroup per CU: the input is
// staged into LDS once per CU, by twice the threads of a 4-wavefront group.
#ifndef LMK_GEMV_NT
#define LMK_GEMV_NT 512
#endif
constexpr int kGemvThreads = LMK_GEMV_NT;

// ---------------------------------------------------------------------------
// helpers
// ---------------------------------------------------------------------------

// Weight loads (quants, block scales, K-format headers and high bits) carry
// the non-temporal hint: every such byte is read once per step.  Measured
// faster for the 8B and 70B matrices (8B Q8_0 step 1.92 -> 1.82 ms, Q4_K /
// Q5_K 2-3 %) but slower for small ones (a 1B model's QKV 4.6 -> 5.5 us), so
// the one-sequence Q8_0 / Q4_0 GEMV takes it only for matrices of at least
// kStreamBytes; the KV cache made attention slower with it and keeps plain
// loads.
typedef int v4i_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int4 ld16_stream(const uint8_t* p) {
    const v4i_t v = __builtin_nontemporal_load((const v4i_t*)p);
    return make_int4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16_stream(const uint4* p) {
    const v4i_t v = __builtin_nontemporal_load((const v4i_t*)p);
    return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}
typedef unsigned int u2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ld8_stream(const void* p) {
    const u2v_t v = __builtin_nontemporal_load((const u2v_t*)p);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ld4_stream(const void* p) {
    return __builtin_nontemporal_load((const uint32_t*)p);
}
constexpr int64_t kStreamBytes = 16ll << 20;   // quant bytes of a matrix that takes the hint
// the same loads without the hint (WNT = false) or with it
template <bool WNT> __device__ __forceinline__ int4 ld16_w(const uint8_t* p) {
    if constexpr (WNT) return ld16_stream(p);
    const v4i_t v = *(const v4i_t*)p;
    return make_int4(v.x, v.y, v.z, v.w);
}
template <bool WNT> __device__ __forceinline__ uint32_t ld4_w(const void* p) {
    if constexpr (WNT) return ld4_stream(p);
    return *(const uint32_t*)p;
}

__device__ __forceinline__ float h2f(uint16_t h) {
    return __half2float(__ushort_as_half(h));
}

// Sum over aligned groups of N lanes (N = 8, 16, 32 or 64), the result in
// every lane of the group, without an LDS round trip: DPP moves inside a quad
// (xor 1, xor 2), the mirrors inside each half row and row (8, 16 lanes), then
// gfx950's row and half-wave swaps (v_permlane16_swap: lane l <-> l ^ 16,
// v_permlane32_swap: l <-> l ^ 32).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 8 || N == 16 || N == 32 || N == 64, "group of 8, 16, 32 or 64 lanes");
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
    if (N >= 16) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
    if (N >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    if (N >= 64) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return v;
}
// The four rows (16 lanes each) of x, each broadcast to every lane: out[r]
// in lane l = x in lane 16 r + l % 16.  v_permlane16_swap of x with itself
// gives rows (0, 0, 2, 2) and (1, 1, 3, 3); v_permlane32_swap of each of
// those with itself splits them into single rows.
__device__ __forceinline__ void row_bcast4(uint32_t x, uint32_t (&out)[4]) {
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(a[0], a[0], false, false);
    const auto c = __builtin_amdgcn_permlane32_swap(a[1], a[1], false, false);
    out[0] = b[0];
    out[1] = c[0];
    out[2] = b[1];
    out[3] = c[1];
}
// Rows (0, 0, 2, 2) and (1, 1, 3, 3) of x: out[0] in lane l = x in lane
// 32 (l / 32) + l % 16, out[1] = x in lane 32 (l / 32) + 16 + l % 16.
__device__ __forceinline__ void row_bcast2(uint32_t x, uint32_t (&out)[2]) {
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    out[0] = a[0];
    out[1] = a[1];
}
// max / sum with the lane 16 and 32 apart (all lanes get the result)
__device__ __forceinline__ float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// (value, index) maximum with the lowest index winning ties
__device__ __forceinline__ void better(float& bv, int& bi, float v, int i) {
    if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

// (value, index) maximum over aligned groups of N lanes (N = 16 or 64), the
// result in every lane of the group: the steps of group_sum, applied to the
// value and its index alike.
template <int N>
__device__ __forceinline__ void group_argmax(float& bv, int& bi) {
    static_assert(N == 16 || N == 64, "group of 16 or 64 lanes");
    #define LMK_DPP_STEP(ctrl)                                                                         \
        {                                                                                              \
            const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(bv), ctrl, 0xF, 0xF, false)); \
            const int oi = __builtin_amdgcn_mov_dpp(bi, ctrl, 0xF, 0xF, false);                        \
            better(bv, bi, ov, oi);                                                                    \
        }
    LMK_DPP_STEP(0xB1)    // quad_perm [1,0,3,2]
    LMK_DPP_STEP(0x4E)    // quad_perm [2,3,0,1]
    LMK_DPP_STEP(0x141)   // row_half_mirror
    LMK_DPP_STEP(0x140)   // row_mirror
    #undef LMK_DPP_STEP
    if (N == 64) {
        const auto v16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
        const auto i16 = __builtin_amdgcn_permlane16_swap((uint32_t)bi, (uint32_t)bi, false, false);
        bv = __uint_as_float(v16[0]);
        bi = (int)i16[0];
        better(bv, bi, __uint_as_float(v16[1]), (int)i16[1]);
        const auto v32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(bv), __float_as_uint(bv), false, false);
        const auto i32 = __builtin_amdgcn_permlane32_swap((uint32_t)bi, (uint32_t)bi, false, false);
        bv = __uint_as_float(v32[0]);
        bi = (int)i32[0];
        better(bv, bi, __uint_as_float(v32[1]), (int)i32[1]);
    }
}

// Activations enter the integer dot products as 24-bit fixed point: per
// 32-column block b, X_i = rint(x_i * 127*2^16 / max|x_b|), split into three
// balanced signed 8-bit digits X = D2*2^16 + D1*2^8 + D0 (two's-complement
// bytes: D0 = low byte of X, D1 = low byte of (X+128)>>8, D2 = (X+2^15+128)>>16).
// sum_i q_i x_i = sx_b * (2^16 S2 + 2^8 S1 + S0), S_k = sum_i q_i D_k,i, with
// sx_b = max|x_b| / (127*2^16).  The S_k are exact int32 sums of v_dot4 products;
// the only rounding is X's (relative 2^-24 of the block maximum) and the fp32
// combination, the same order as an fp32 dot product.
__device__ __forceinline__ int sdot4(int a, int b, int c) { return __builtin_amdgcn_sdot4(a, b, c, false); }

__device__ __forceinline__ float combine_digits(int s0, int s1, int s2) {
    return fmaf((float)(s2 * 256 + s1), 256.f, (float)s0);
}

// Q8_0 block: A = elements 0..15, B = 16..31 (int8); D = the block's digit
// planes [D0 0..15][D0 16..31][D1 ..][D1 ..][D2 ..][D2 ..] as int4s.
__device__ __forceinline__ float dot_q8(const int4 A, const int4 B, const int4* D) {
    const int4 e0 = D[0], e1 = D[1], f0 = D[2], f1 = D[3], g0 = D[4], g1 = D[5];
    int s0 = sdot4(A.x, e0.x, 0), s1 = sdot4(A.x, f0.x, 0), s2 = sdot4(A.x, g0.x, 0);
    s0 = sdot4(A.y, e0.y, s0); s1 = sdot4(A.y, f0.y, s1); s2 = sdot4(A.y, g0.y, s2);
    s0 = sdot4(A.z, e0.z, s0); s1 = sdot4(A.z, f0.z, s1); s2 = sdot4(A.z, g0.z, s2);
    s0 = sdot4(A.w, e0.w, s0); s1 = sdot4(A.w, f0.w, s1); s2 = sdot4(A.w, g0.w, s2);
    s0 = sdot4(B.x, e1.x, s0); s1 = sdot4(B.x, f1.x, s1); s2 = sdot4(B.x, g1.x, s2);
    s0 = sdot4(B.y, e1.y, s0); s1 = sdot4(B.y, f1.y, s1); s2 = sdot4(B.y, g1.y, s2);
    s0 = sdot4(B.z, e1.z, s0); s1 = sdot4(B.z, f1.z, s1); s2 = sdot4(B.z, g1.z, s2);
    s0 = sdot4(B.w, e1.w, s0); s1 = sdot4(B.w, f1.w, s1); s2 = sdot4(B.w, g1.w, s2);
    return combine_digits(s0, s1, s2);
}

// Q4_0 block: 16 bytes, byte j = element j (low nibble) | element j+16 (high).
// The nibbles n = q + OFF enter the dot products unsigned; T = the block's
// digit sums (T0, T1, T2) remove the offset (Q4_0: OFF = 8; the Q4_K
// sub-blocks, regrouped into this order, have OFF = 0: sum n x).
template <int OFF = 8>
__device__ __forceinline__ float dot_q4(const int4 A, const int4* D, const int4 T) {
    const int4 e0 = D[0], e1 = D[1], f0 = D[2], f1 = D[3], g0 = D[4], g1 = D[5];
    const int w[4] = {A.x, A.y, A.z, A.w};
    const int E0[4] = {e0.x, e0.y, e0.z, e0.w}, E1[4] = {e1.x, e1.y, e1.z, e1.w};
    const int F0[4] = {f0.x, f0.y, f0.z, f0.w}, F1[4] = {f1.x, f1.y, f1.z, f1.w};
    const int G0[4] = {g0.x, g0.y, g0.z, g0.w}, G1[4] = {g1.x, g1.y, g1.z, g1.w};
    int s0 = -OFF * T.x, s1 = -OFF * T.y, s2 = -OFF * T.z;
    #pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int lo = w[u] & 0x0F0F0F0F, hi = (int)(((unsigned)w[u] >> 4) & 0x0F0F0F0Fu);
        s0 = sdot4(lo, E0[u], s0); s1 = sdot4(lo, F0[u], s1); s2 = sdot4(lo, G0[u], s2);
        s0 = sdot4(hi, E1[u], s0); s1 = sdot4(hi, F1[u], s1); s2 = sdot4(hi, G1[u], s2);
    }
    return combine_digits(s0, s1, s2);
}

// Q4_K sub-block j (0..7) of a super-block: its 6-bit scale and min from the
// 16-byte header h (x = fp16 d | fp16 dmin << 16; y, z, w = packed bytes
// p0..p3, p4..p7, p8..p11).  Sub-blocks 0..3: scale = p[j] & 63, min =
// p[j+4] & 63; sub-blocks 4..7: the low 4 bits of both in p[j+4] (scale low
// nibble, min high nibble), the top 2 bits in p[j-4] (scale) and p[j] (min).
// Returns ds = d * scale and dm = dmin * min (both exact in fp32).
__device__ __forceinline__ void q4k_scale_min(const int4 h, int j, float& ds, float& dm) {
    const int sh = 8 * (j & 3);
    const uint32_t by = ((uint32_t)h.y >> sh) & 255u, bz = ((uint32_t)h.z >> sh) & 255u,
                   bw = ((uint32_t)h.w >> sh) & 255u;
    const uint32_t sc = j < 4 ? (by & 63u) : ((bw & 15u) | ((by >> 6) << 4));
    const uint32_t mn = j < 4 ? (bz & 63u) : ((bw >> 4) | ((bz >> 6) << 4));
    ds = h2f((uint16_t)((uint32_t)h.x & 0xFFFFu)) * (float)sc;
    dm = h2f((uint16_t)((uint32_t)h.x >> 16)) * (float)mn;
}

// Q5_K sub-block (32 weights): A = low nibbles in the Q4_0 order, H = the
// fifth bits (element 4u+k's at bit 8k + u, element 16+4u+k's at bit
// 8k + 4 + u).  Returns sum q x over the sub-block, q = nibble | bit << 4
// (0..31, unsigned in the dot products).
__device__ __forceinline__ float dot_q5(const int4 A, const uint32_t H, const int4* D) {
    const int4 e0 = D[0], e1 = D[1], f0 = D[2], f1 = D[3], g0 = D[4], g1 = D[5];
    const int w[4] = {A.x, A.y, A.z, A.w};
    const int E0[4] = {e0.x, e0.y, e0.z, e0.w}, E1[4] = {e1.x, e1.y, e1.z, e1.w};
    const int F0[4] = {f0.x, f0.y, f0.z, f0.w}, F1[4] = {f1.x, f1.y, f1.z, f1.w};
    const int G0[4] = {g0.x, g0.y, g0.z, g0.w}, G1[4] = {g1.x, g1.y, g1.z, g1.w};
    int s0 = 0, s1 = 0, s2 = 0;
    #pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int lo = (int)(((uint32_t)w[u] & 0x0F0F0F0Fu) | ((H << (4 - u)) & 0x10101010u));
        const int hi = (int)((((uint32_t)w[u] >> 4) & 0x0F0F0F0Fu) | ((H >> u) & 0x10101010u));
        s0 = sdot4(lo, E0[u], s0); s1 = sdot4(lo, F0[u], s1); s2 = sdot4(lo, G0[u], s2);
        s0 = sdot4(hi, E1[u], s0); s1 = sdot4(hi, F1[u], s1); s2 = sdot4(hi, G1[u], s2);
    }
    return combine_digits(s0, s1, s2);
}

// Q6_K block (32 weights, two 16-weight sub-blocks): A = low nibbles in the
// Q4_0 order, Hb = the high parts (word x: elements 0..15, y: 16..31; element
// 4u+k's two bits at bit 8k + 2u).  q = low | high << 4 (0..63) enters the dot
// products unsigned; the sub-blocks' digit sums T0 (elements 0..15), T1
// (16..31) remove the 32 offset.  lo / hi = sum (q - 32) x over each sub-block.
__device__ __forceinline__ void dot_q6(const int4 A, const uint2 Hb, const int4* D, const int4 T0,
                                       const int4 T1, float& lo, float& hi) {
    const int4 e0 = D[0], e1 = D[1], f0 = D[2], f1 = D[3], g0 = D[4], g1 = D[5];
    const int w[4] = {A.x, A.y, A.z, A.w};
    const int E0[4] = {e0.x, e0.y, e0.z, e0.w}, E1[4] = {e1.x, e1.y, e1.z, e1.w};
    const int F0[4] = {f0.x, f0.y, f0.z, f0.w}, F1[4] = {f1.x, f1.y, f1.z, f1.w};
    const int G0[4] = {g0.x, g0.y, g0.z, g0.w}, G1[4] = {g1.x, g1.y, g1.z, g1.w};
    int a0 = -32 * T0.x, a1 = -32 * T0.y, a2 = -32 * T0.z;
    int b0 = -32 * T1.x, b1 = -32 * T1.y, b2 = -32 * T1.z;
    #pragma unroll
    for (int u = 0; u < 4; ++u) {
        // move bits 8k + 2u, 8k + 2u + 1 to 8k + 4, 8k + 5
        const uint32_t hl = u < 2 ? Hb.x << (4 - 2 * u) : Hb.x >> (2 * u - 4);
        const uint32_t hh = u < 2 ? Hb.y << (4 - 2 * u) : Hb.y >> (2 * u - 4);
        const int vl = (int)(((uint32_t)w[u] & 0x0F0F0F0Fu) | (hl & 0x30303030u));
        const int vh = (int)((((uint32_t)w[u] >> 4) & 0x0F0F0F0Fu) | (hh & 0x30303030u));
        a0 = sdot4(vl, E0[u], a0); a1 = sdot4(vl, F0[u], a1); a2 = sdot4(vl, G0[u], a2);
        b0 = sdot4(vh, E1[u], b0); b1 = sdot4(vh, F1[u], b1); b2 = sdot4(vh, G1[u], b2);
    }
    lo = combine_digits(a0, a1, a2);
    hi = combine_digits(b0, b1, b2);
}

// Sum over a workgroup of NW wavefronts (red: NW floats of LDS).
template <int NW = kWaves>
__device__ __forceinline__ float block_sum(float v, float* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = 0.f;
    #pragma unroll
    for (int w = 0; w < NW; ++w) t += red[w];
    return t;
}

// ---------------------------------------------------------------------------
// dequant-GEMV with fused prologue / epilogue
// ---------------------------------------------------------------------------

// Reductions over the 8 lanes i..i|7 with DPP moves (no LDS round trip):
// xor 1 and xor 2 inside a quad, then the mirror inside each half row (lane
// i <-> 7 - i) brings the other quad's result.
__device__ __forceinline__ float max8(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));  // quad_perm [1,0,3,2]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));  // quad_perm [2,3,0,1]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false))); // row_half_mirror
    return v;
}
__device__ __forceinline__ int sum4(int v) {
    v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
    v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
    return v;
}
__device__ __forceinline__ int sum8(int v) {
    v = sum4(v);
    v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
    return v;
}

// Four consecutive activations (columns i..i+3 of a 32-column block) -> their
// three digit bytes; the block maximum comes from the 8 lanes sharing the block.
// sums: 0 none; 1 the block's digit sums at dsum[b]; 2 the sums of its two
// 16-column halves at dsum[2b], dsum[2b+1].
__device__ __forceinline__ void stage_digits(float4 v, int i, int K, int8_t* xq, float* xsc, int4* dsum,
                                             int sums) {
    const float m = max8(fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    if (i >= K) return;
    const float f = m > 0.f ? 8323072.0f / m : 0.f;       // 127 * 2^16 / max|x_b|
    const int X[4] = {(int)rintf(v.x * f), (int)rintf(v.y * f), (int)rintf(v.z * f), (int)rintf(v.w * f)};
    uint32_t w0 = 0, w1 = 0, w2 = 0;
    int t0 = 0, t1 = 0, t2 = 0;
    #pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int x1 = (X[e] + 128) >> 8, x2 = (x1 + 128) >> 8;
        w0 |= (uint32_t)(X[e] & 255) << (8 * e);
        w1 |= (uint32_t)(x1 & 255) << (8 * e);
        w2 |= (uint32_t)(x2 & 255) << (8 * e);
        t0 += (int)(int8_t)(X[e] & 255);
        t1 += (int)(int8_t)(x1 & 255);
        t2 += x2;
    }
    const int b = i >> 5, j = (i >> 2) & 7;
    int* dst = (int*)(xq + b * 96);
    dst[j] = (int)w0;
    dst[8 + j] = (int)w1;
    dst[16 + j] = (int)w2;
    if (j == 0) xsc[b] = m * (1.0f / 8323072.0f);
    if (sums == 1) {
        t0 = sum8(t0);
        t1 = sum8(t1);
        t2 = sum8(t2);
        if (j == 0) dsum[b] = make_int4(t0, t1, t2, 0);
    } else if (sums == 2) {
        t0 = sum4(t0);
        t1 = sum4(t1);
        t2 = sum4(t2);
        if ((j & 3) == 0) dsum[2 * b + (j >> 2)] = make_int4(t0, t1, t2, 0);
    }
}


// Cross-workgroup hand-off within one launch.  Each XCD has its own L2,
// which is not coherent with the others', and an acquire or release at device
// scope makes the compiler write back (buffer_wbl2) and invalidate
// (buffer_inv) that whole L2 at every use: once per workgroup this cost the
// 4096-position batch-4 attention more than half its time.  The hand-offs
// below get the same ordering from the memory operations themselves instead:
//   * the data crosses in device-coherent stores and loads (relaxed atomics
//     at device scope, which the hardware issues with the sc1 bit: the store
//     is written through to memory-side coherence, the load is not served
//     from a non-coherent cache);
//   * every wavefront waits for its stores to complete (vmcnt(0)) and the
//     workgroup meets at a barrier before one thread counts its arrival, so
//     the data is visible device-wide before the count moves;
//   * the caller that completes the count reads the data only after the
//     count's returned value and a barrier, so those loads are issued after
//     every earlier arrival was counted.
// The barriers also keep the compiler from moving these memory operations
// across the count.
__device__ __forceinline__ void st_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_dev(const int* p) {
    return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// two floats at an 8-byte aligned address, device-coherent
__device__ __forceinline__ void st_dev2(float* p, float x, float y) {
    const uint64_t v = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
    __hip_atomic_store((uint64_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_dev2(const float* p) {
    const uint64_t v = __hip_atomic_load((uint64_t*)const_cast<float*>(p), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)v), __uint_as_float((uint32_t)(v >> 32)));
}
// this wavefront's outstanding memory operations have completed (gfx9 vmcnt(0))
__device__ __forceinline__ void drain_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// one arrival of n on a device-scope count; true for the caller that makes it
// n, which also resets it to zero for the next launch.  One thread calls it,
// between the barriers described above.
__device__ __forceinline__ bool count_arrive(int* c, int n) {
    if (__hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != n - 1) return false;
    __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// ---------------------------------------------------------------------------
// split-context attention
// ---------------------------------------------------------------------------
// Counts one more finished chunk of a (sequence, KV head) whose n_act chunks
// publish partial states; true for the caller that completes the count (it
// then merges).  Two levels, so that at most kCntGroup atomics meet on one
// line: chunks count into their group's line, the chunk completing a group
// counts into line 0.  Whoever completes a count resets it for the next launch.
// One thread calls it, after its workgroup's partial stores have completed
// (the hand-off above; the second level is reached only after the first
// level's count has returned).
__device__ __forceinline__ bool chunk_arrive(int* cnt, int chunk, int n_act) {
    const int grp = chunk / kCntGroup, n_grp = (n_act + kCntGroup - 1) / kCntGroup;
    const int in_grp = min(kCntGroup, n_act - grp * kCntGroup);
    if (!count_arrive(cnt + (1 + grp) * kCntStride, in_grp)) return false;
    return n_grp == 1 || count_arrive(cnt, n_grp);
}

// Log-sum-exp merge of the n_act chunk states of the G query heads of one KV
// head (the split softmax of FlashDecoding-style attention; the pages' GQA
// decode attention computes softmax(q K^T / sqrt(hd)) V over keys 0..pos):
//   out[j][d] = sum_c o_c[d] e^(m_c - M) / sum_c l_c e^(m_c - M),  M = max_c m_c,
// where chunk c's record (part(j) + c * (HD + 2)) holds its unnormalised
// o[HD] = sum_t e^(s_t - m_c) v_t, then m_c and l_c = sum_t e^(s_t - m_c).
// The merge is latency-bound, so it is laid out for memory-level parallelism:
// a thread per (partition of the chunks, query head, 4 dimensions), each batch
// of kB chunks loaded in full before the first is used, the partitions combined
// in LDS.  ld2(p) returns the two floats at the 8-byte aligned p, device-
// coherently; st4(i, v) writes out[i..i+3] (i = j * HD + d).  Cs: LDS scratch,
// kBlock x 6 floats.  Every thread of the workgroup calls it (one barrier).
template <int HD, class Part, class Ld2, class St4>
__device__ __forceinline__ void merge_chunk_states(int G, int n_act, Part part, Ld2 ld2, St4 st4,
                                                   float (*Cs)[6]) {
    constexpr int kB = 8;                      // chunks per batch of loads
    constexpr int64_t stride = HD + 2;
    const int tid = threadIdx.x;
    const int n_out = G * HD / 4;              // float4 outputs (at most kBlock)
    const int P = kBlock / n_out;              // partitions of the chunks
    const int p = tid / n_out, r = tid % n_out;
    const int j = r / (HD / 4), d4 = (r % (HD / 4)) * 4;
    const float* ph = part(j);
    float M = -FLT_MAX, L = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
    for (int base = p < P ? p * kB : n_act; base < n_act; base += P * kB) {
        float2 ml[kB], o01[kB], o23[kB];
        #pragma unroll
        for (int u = 0; u < kB; ++u) {
            const float* pc = ph + min(base + u, n_act - 1) * stride;
            ml[u] = ld2(pc + HD);
            o01[u] = ld2(pc + d4);
            o23[u] = ld2(pc + d4 + 2);
        }
        float bm = M;
        #pragma unroll
        for (int u = 0; u < kB; ++u)
            if (base + u < n_act) bm = fmaxf(bm, ml[u].x);
        const float rs = __expf(M - bm);
        L *= rs;
        #pragma unroll
        for (int k = 0; k < 4; ++k) O[k] *= rs;
        #pragma unroll
        for (int u = 0; u < kB; ++u)
            if (base + u < n_act) {
                const float e = __expf(ml[u].x - bm);
                L = fmaf(ml[u].y, e, L);
                O[0] = fmaf(o01[u].x, e, O[0]);
                O[1] = fmaf(o01[u].y, e, O[1]);
                O[2] = fmaf(o23[u].x, e, O[2]);
                O[3] = fmaf(o23[u].y, e, O[3]);
            }
        M = bm;
    }
    Cs[tid][0] = M;
    Cs[tid][1] = L;
    #pragma unroll
    for (int k = 0; k < 4; ++k) Cs[tid][2 + k] = O[k];
    __syncthreads();
    if (p != 0) return;
    float Mt = M;
    for (int q = 1; q < P; ++q) Mt = fmaxf(Mt, Cs[q * n_out + r][0]);
    float Lt = 0.f, Ot[4] = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < P; ++q) {
        const float* c = Cs[q * n_out + r];
        if (c[0] == -FLT_MAX) continue;        // a partition that holds no chunk
        const float e = __expf(c[0] - Mt);
        Lt = fmaf(c[1], e, Lt);
        #pragma unroll
        for (int k = 0; k < 4; ++k) Ot[k] = fmaf(c[2 + k], e, Ot[k]);
    }
    const float inv = 1.f / Lt;
    st4(j * HD + d4, make_float4(Ot[0] * inv, Ot[1] * inv, Ot[2] * inv, Ot[3] * inv));
}

}  // namespace lmk
