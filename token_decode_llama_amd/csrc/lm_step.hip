// lm_step.hip - one batch-1 decode step as a single persistent kernel (gfx950).
//
// The step is the operator chain of the C/CUDA Llama engine page
// (rskf.cn/news/15116, section 4.4: single-token GEMV, RMSNorm fused with its
// gain, RoPE from a precomputed sin/cos table fused with the producer,
// SwiGLU fused with the FC product, softmax with the causal mask folded in):
// per layer QKV -> GQA attention -> Wo (+ residual) -> gate/up (SwiGLU) ->
// down (+ residual), then the final norm, the LM head and the argmax.  Each
// of these is a "phase"; every GEMV input depends on all outputs of the
// phase before it.
//
// MI355X design: one workgroup per CU for the whole step.
//  * Weight streaming is decoupled from the dependency chain.  The weights a
//    CU multiplies are fixed in advance (an interleaved share of every
//    matrix's 4-row groups), so four producer wavefronts stream them, phase
//    after phase, into a ring of 9 KB LDS slots and never wait for
//    activations.  A slot holds one tile: 4 rows x up to 64 Q8_0 (128 Q4_0)
//    blocks, contiguous in HBM (a tile-major copy made at load time), so a
//    tile is one coalesced read.
//  * Four consumer wavefronts follow the dependency chain: at the start of
//    a phase they stage the input vector (RMSNorm folded in) as integer
//    digits in LDS, then take their tiles from the ring, accumulate the four
//    rows' dot products and run the phase's epilogue.  Between phases they
//    cross a grid-wide barrier; meanwhile the producers keep filling the
//    ring, so the HBM stream does not stop at phase boundaries.
//  * Data that crosses CUs inside the step (x, q, o, h, the new K/V row,
//    attention and argmax partials, barrier counters) moves through
//    device-coherent relaxed atomic loads and stores; a wavefront waits for
//    its own stores to complete before it signals.  No cache writeback or
//    invalidate is needed.
//  * Attention is a phase of its own: one item per (KV head, 64-position
//    chunk) spread over the CUs; the last chunk of a KV head merges the
//    partial softmax states (log-sum-exp).
// Every wait is bounded: a timeout sets an error flag and all wavefronts
// leave the kernel.
#include "lm_device.h"
#include "lm_step.h"

namespace lmk {

constexpr int kNP = 4;                       // producer wavefronts
constexpr int kNC = 4;                       // consumer wavefronts
constexpr int kStepThreads = 64 * (kNP + kNC);
constexpr int kCT = 64 * kNC;                // consumer threads
constexpr int kLoadsPerLane = kStepSlotBytes / 16 / 64;   // 16-byte loads per lane per tile
constexpr int kSpinLds = 40000000;           // bounded waits on LDS flags
constexpr int kSpinDev = 4000000;            // bounded waits on device counters
constexpr int kAttnCh = 64;                  // positions per attention item
constexpr int kMaxG = 8;                     // query heads per KV head

static_assert(kLoadsPerLane * 64 * 16 == kStepSlotBytes, "a slot is whole 1 KB wavefront loads");
static_assert(sizeof(int) * 2 * kStepMaxSlots + 64 + 12 * kNC + 8 * kPartBufs +
                  4 * kPartBufs * kNC * kTileRows <= kStepCtlBytes, "control block fits");

template <int QT> struct TileNbk { static constexpr int value = kTileBlocksQ8; };
template <> struct TileNbk<kQ4_0> { static constexpr int value = kTileBlocksQ4; };

// ---- device memory through address-space-1 (global) pointers ---------------
// Pointers read from the argument block are generic to the compiler; the casts
// below make every access a global (not flat) instruction, so LDS waits
// (lgkmcnt) never wait on device memory.
#define LMK_G __attribute__((address_space(1)))
typedef int v4i_g __attribute__((ext_vector_type(4)));
typedef float v4f_g __attribute__((ext_vector_type(4)));
typedef unsigned int v2u_g __attribute__((ext_vector_type(2)));
template <class T> __device__ __forceinline__ LMK_G T* gp(T* p) { return (LMK_G T*)p; }
template <class T> __device__ __forceinline__ const LMK_G T* gp(const T* p) { return (const LMK_G T*)p; }

__device__ __forceinline__ int4 ldg16(const void* p) {
    const v4i_g v = *(const LMK_G v4i_g*)p;
    return make_int4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ int4 ldg16_nt(const void* p) {
#if LMK_WEIGHT_NT
    const v4i_g v = __builtin_nontemporal_load((const LMK_G v4i_g*)p);
#else
    const v4i_g v = *(const LMK_G v4i_g*)p;
#endif
    return make_int4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ldgf4(const float* p) {
    const v4f_g v = *(const LMK_G v4f_g*)p;
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float ldgf(const float* p) { return *gp(p); }

// ---- device-coherent traffic --------------------------------------------------
__device__ __forceinline__ float ldc(const float* p) {
    return __hip_atomic_load(gp(const_cast<float*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(float* p, float v) {
    __hip_atomic_store(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ldc32(const void* p) {
    return __hip_atomic_load(gp((uint32_t*)const_cast<void*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc32(void* p, uint32_t v) {
    __hip_atomic_store(gp((uint32_t*)p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ldc64(const void* p) {
    return __hip_atomic_load(gp((uint64_t*)const_cast<void*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t addc32(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(gp(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// this wavefront's outstanding memory operations have completed (gfx9 vmcnt(0))
__device__ __forceinline__ void drain_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// this wavefront's outstanding LDS operations have completed (lgkmcnt(0) only)
__device__ __forceinline__ void drain_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// ---- debug timestamps (constant 100 MHz clock) -------------------------------
__device__ __forceinline__ void trace_at(const StepArgs* __restrict__ a, int ph, int word) {
    if (a->trace) *gp(a->trace + ((int64_t)blockIdx.x * (5 * a->L + 1) + ph) * kTraceWords + word) =
        (uint64_t)__builtin_amdgcn_s_memrealtime();
}

// ---- LDS flags, read uniformly --------------------------------------------------
__device__ __forceinline__ int lds_get(const int* p) {
    return __builtin_amdgcn_readfirstlane(__atomic_load_n(p, __ATOMIC_RELAXED));
}
__device__ __forceinline__ void lds_put(int* p, int v) { __atomic_store_n(p, v, __ATOMIC_RELAXED); }

struct StepCtl {
    int ready[kStepMaxSlots];     // global tile index the slot now holds
    int done[kStepMaxSlots];      // global tile index last released from the slot
    int csync;                    // consumer arrivals (monotonic)
    int gen;                      // grid barriers crossed
    int abort;
    int flag;                     // small broadcasts among the consumers
    float red[kNC];
    float bv[kNC];
    int bi[kNC];
    int pcnt[kPartBufs];          // partial sums stored for the buffer's row group
    int pdone[kPartBufs];         // last row group (cumulative index) finished from the buffer
    float part[kPartBufs][kNC][kTileRows];
};

struct PhaseMat {
    const uint8_t* base;
    TileGeom g;
};

// weighted phases in order: layer l's QKV, Wo, gate/up, down (wp = 4l + t), then the LM head
__device__ __forceinline__ PhaseMat phase_mat(const StepArgs* __restrict__ a, int wp) {
    PhaseMat m;
    if (wp < 4 * a->L) {
        const int l = wp >> 2, t = wp & 3;
        m.base = a->tiles + (int64_t)l * a->layer_stride + a->mat_off[t];
        m.g = a->geo[t];
    } else {
        m.base = a->lm_tiles;
        m.g = a->geo[4];
    }
    return m;
}

// row groups of a matrix that this CU owns: cu, cu + G, cu + 2G, ...
__device__ __forceinline__ int my_groups(int ng, int cu, int G) { return ng > cu ? (ng - cu + G - 1) / G : 0; }

// ============================================================================
// producer: this CU's tiles of every weighted phase, in order, into the ring
// ============================================================================
// The tiles are read with direct-to-LDS loads (gfx950 global_load_lds_dwordx4:
// each lane's 16 bytes land at slot + 16 * lane), so nothing is staged in
// registers; kProdDepth tiles per wavefront are in flight, and a tile is
// marked ready once the in-order load counter shows its loads have landed.
// The LDS flags are read and written with inline ds instructions, which the
// compiler does not order behind the outstanding direct-to-LDS loads.
constexpr int kProdDepth = 3;

__device__ __forceinline__ int lds_get_asm(const int* p) {
    int v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"((uint32_t)(uintptr_t)p) : "memory");
    return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ void lds_put_asm(int* p, int v) {
    asm volatile("ds_write_b32 %0, %1" ::"v"((uint32_t)(uintptr_t)p), "v"(v) : "memory");
}

template <int QT>
__device__ void producer(const StepArgs* __restrict__ a, uint8_t* ring, StepCtl* C, int wave, int lane) {
    const int G = gridDim.x, cu = blockIdx.x, NS = a->ring_slots;
    const int n_wp = 4 * a->L + 1;
    int wp = 0, pos = 0, n_in = 0;    // cursor: weighted phase, tile within this CU's share of it
    PhaseMat pm = phase_mat(a, 0);
    n_in = my_groups(pm.g.ng, cu, G) * pm.g.nch;
    auto advance = [&](int n) -> bool {
        pos += n;
        while (pos >= n_in) {
            pos -= n_in;
            if (++wp >= n_wp) return false;
            pm = phase_mat(a, wp);
            n_in = my_groups(pm.g.ng, cu, G) * pm.g.nch;
        }
        return true;
    };
    int pend = 0, oldest = 0;         // tiles issued and not yet marked ready (oldest first)
    auto mark_all = [&]() {
        drain_vm();
        for (; pend > 0; --pend, oldest += kNP)
            if (lane == 0) lds_put_asm(&C->ready[oldest % NS], oldest);
    };
    int traced_wp = -1;
    bool more = advance(wave);        // this wavefront's tiles: k = wave, wave + kNP, ...
    for (int k = wave; more; k += kNP) {
        const int s = k % NS;
        if (lds_get_asm(&C->done[s]) != k - NS) {
            mark_all();                                   // never hold landed tiles while waiting
            int spins = 0;
            while (lds_get_asm(&C->done[s]) != k - NS) {
                __builtin_amdgcn_s_sleep(1);
                if (++spins > kSpinLds || lds_get_asm(&C->abort)) {
                    lds_put_asm(&C->abort, 1);
                    return;
                }
            }
        }
        if (wave == 0 && a->trace && wp != traced_wp) {
            traced_wp = wp;
            const int ph = wp < 4 * a->L ? (wp >> 2) * 5 + ((wp & 3) == 0 ? 0 : (wp & 3) + 1) : 5 * a->L;
            if (lane == 0) trace_at(a, ph, 4);
        }
        const int i = pos / pm.g.nch, c = pos - i * pm.g.nch;
        const uint8_t* t = pm.base + (int64_t)(cu + G * i) * pm.g.gbytes + (int64_t)c * pm.g.tfull;
        const int units = c == pm.g.nch - 1 ? pm.g.ulast : pm.g.ufull;
        uint8_t* slot = ring + (int64_t)s * kStepSlotBytes;
        #pragma unroll
        for (int j = 0; j < kLoadsPerLane; ++j) {
            const int u = min(lane + 64 * j, units - 1);  // clamped: always inside the tile
            __builtin_amdgcn_global_load_lds((const LMK_G void*)(t + (uint32_t)u * 16u),
                                             (__attribute__((address_space(3))) void*)(slot + 1024 * j), 16, 0, 0);
        }
        if (pend == 0) oldest = k;
        ++pend;
        if (pend == kProdDepth) {
            // the oldest tile's loads are the first kLoadsPerLane of the outstanding ones
            __builtin_amdgcn_s_waitcnt((((kLoadsPerLane * (kProdDepth - 1)) >> 4) << 14) |
                                       ((kLoadsPerLane * (kProdDepth - 1)) & 15) | 0x0F70);
            if (lane == 0) lds_put_asm(&C->ready[oldest % NS], oldest);
            oldest += kNP;
            --pend;
        }
        more = advance(kNP);
    }
    mark_all();
}

// ============================================================================
// consumers
// ============================================================================
struct Cons {
    const StepArgs* __restrict__ a;
    uint8_t* ring;
    uint8_t* xr;          // input digits / attention scratch
    StepCtl* C;
    int cw, lane, ct;     // consumer wavefront, lane, consumer thread
    uint32_t epoch;
    int nsync = 0;
    bool ok = true;
    uint64_t t_wait = 0, t_comp = 0, n_tiles = 0;   // debug trace: consumer-0 cycles per phase

    __device__ Cons(const StepArgs* aa, uint8_t* r, uint8_t* x, StepCtl* c, int w, int l)
        : a(aa), ring(r), xr(x), C(c), cw(w), lane(l), ct(w * 64 + l), epoch(0) {}

    __device__ bool fail() {
        lds_put(&C->abort, 1);
        ok = false;
        return false;
    }

    // Every consumer wavefront arrives here; its LDS writes (and, with
    // drain_dev, its device stores) have completed when it arrives.
    __device__ bool sync(bool drain_dev) {
        if (drain_dev) drain_vm();
        drain_lds();
        ++nsync;
        if (lane == 0) __hip_atomic_fetch_add(&C->csync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int want = kNC * nsync;
        int spins = 0;
        while (lds_get(&C->csync) < want) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLds || lds_get(&C->abort)) return fail();
        }
        return true;
    }

    // Grid-wide barrier after phase p: one count per XCD group of workgroups,
    // the last arrival of a group adds to the phase's global count.  Counts
    // keep growing from launch to launch (round = epoch + 1).
    __device__ bool grid_barrier(int p) {
        if (!sync(true)) return false;
        if (cw == 0 && lane == 0) trace_at(a, p, 3);
        if (cw == 0 && lane == 0) {
            const int G = gridDim.x, NX = min(8, G);
            uint32_t* b = a->bar + (int64_t)p * kBarStride;
            const int x = blockIdx.x % NX;
            const uint32_t per = (uint32_t)((G - x + NX - 1) / NX);
            const uint32_t round = epoch + 1u;
            const uint32_t old = addc32(b + 32 * (1 + x), 1u);
            if (old == per * round - 1u) addc32(b, 1u);
            int spins = 0;
            bool good = true;
            while ((int32_t)(ldc32(b) - (uint32_t)NX * round) < 0) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins > kSpinDev || ldc32(a->err) != 0u) { good = false; break; }
            }
            if (!good) {
                stc32(a->err, 1u);
                lds_put(&C->abort, 1);
            }
            lds_put(&C->gen, p + 1);
        }
        int spins = 0;
        while (lds_get(&C->gen) < p + 1) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLds || lds_get(&C->abort)) return fail();
        }
        if (lds_get(&C->abort)) return fail();
        return true;
    }

    __device__ bool wait_tile(int k) {
        const int s = k % a->ring_slots;
        if (lds_get(&C->ready[s]) == k) return true;
        int spins = 0;
        while (lds_get(&C->ready[s]) != k) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLds || lds_get(&C->abort)) return fail();
        }
        return true;
    }
    __device__ void release_tile(int k) {
        drain_lds();
        if (lane == 0) lds_put(&C->done[k % a->ring_slots], k);
    }
};

// ---- phase prologue: the input vector as integer digits in LDS -------------
// The input is a device-coherent fp32 vector, or (emb) an fp16 embedding row
// that CU 0 also writes out as the residual stream x.  With a gain g the
// digits are of x . g and the returned factor 1/sqrt(mean(x^2) + eps)
// multiplies each finished dot product (RMSNorm).
template <int QT>
__device__ float stage_input(Cons& cs, const float* src, const uint16_t* emb, const float* gain, int K,
                             float* x_out) {
    constexpr int NB = 8;               // float4s per thread whose loads are in flight together
    const int nb = K >> 5;
    int8_t* xq = (int8_t*)cs.xr;
    float* xsc = (float*)(xq + (int64_t)nb * 96);
    int4* dsum = (int4*)(xsc + ((nb + 3) & ~3));
    float ss = 0.f;
    for (int base = 0; base < K; base += kCT * 4 * NB) {
        float4 v[NB], gv[NB];
        // every load of the batch first (the device-coherent loads are not
        // reordered by the compiler: issuing them together keeps one round trip)
        #pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int i = base + (u * kCT + cs.ct) * 4;
            const int ic = min(i, K - 4);
            if (emb) {
                const v2u_g raw = *(const LMK_G v2u_g*)(emb + ic);
                v[u].x = h2f((uint16_t)(raw.x & 0xFFFF));
                v[u].y = h2f((uint16_t)(raw.x >> 16));
                v[u].z = h2f((uint16_t)(raw.y & 0xFFFF));
                v[u].w = h2f((uint16_t)(raw.y >> 16));
            } else {
                const uint64_t lo = ldc64(src + ic), hi = ldc64(src + ic + 2);
                v[u].x = __uint_as_float((uint32_t)lo);
                v[u].y = __uint_as_float((uint32_t)(lo >> 32));
                v[u].z = __uint_as_float((uint32_t)hi);
                v[u].w = __uint_as_float((uint32_t)(hi >> 32));
            }
            if (gain) gv[u] = ldgf4(gain + ic);
        }
        #pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int i = base + (u * kCT + cs.ct) * 4;
            if (base + u * kCT * 4 >= K) break;          // uniform: no column of this piece is inside K
            float4 x = v[u];
            if (emb && x_out && i < K) {
                stc(x_out + i, x.x);
                stc(x_out + i + 1, x.y);
                stc(x_out + i + 2, x.z);
                stc(x_out + i + 3, x.w);
            }
            if (gain) {
                if (i < K) {
                    ss = fmaf(x.x, x.x, ss);
                    ss = fmaf(x.y, x.y, ss);
                    ss = fmaf(x.z, x.z, ss);
                    ss = fmaf(x.w, x.w, ss);
                }
                x.x *= gv[u].x;
                x.y *= gv[u].y;
                x.z *= gv[u].z;
                x.w *= gv[u].w;
            }
            stage_digits(x, i, K, xq, xsc, dsum, QT == kQ4_0);
        }
    }
    if (gain) {
        ss = wave_sum(ss);
        if (cs.lane == 0) cs.C->red[cs.cw] = ss;
    }
    if (!cs.sync(false)) return 1.f;
    if (!gain) return 1.f;
    float t = 0.f;
    #pragma unroll
    for (int w = 0; w < kNC; ++w) t += cs.C->red[w];
    return 1.0f / sqrtf(t / (float)K + cs.a->eps);
}

// ---- one tile on the matrix cores ------------------------------------------
// v_mfma_i32_4x4x4i8 computes 16 independent 4x4x4 products; lane l = 4m + j
// supplies A_m[j][0..3] and B_m[0..3][j] and receives D_m[0..3][j].  Product
// m here is (input block l / 16 of four, weight row l mod 16): A_m row i =
// digit i of the input's block (row 3 repeats digit 0 and is ignored), B_m
// column j = the weight row, and eight products over k = 4c..4c+3 (c = 0..7)
// accumulate the whole 32-column block.  Lane l ends with the three exact
// digit sums of its (row, block) pair, combines them and scales them by
// weight scale x input block scale into its fp32 accumulator; the four
// lanes of a row (l, l+16, l+32, l+48) are added at the end of the row group.
typedef int v4i_mf __attribute__((ext_vector_type(4)));

template <int QT>
__device__ __forceinline__ void tile_mfma(const uint8_t* T, int nbk, int b0, const int8_t* xq, const float* xsc,
                                          const int4* dsum, int lane, float& acc) {
    constexpr int QBB = QT == kQ8_0 ? 512 : 256;      // quant bytes of one block of 16 rows
    const uint16_t* sc = (const uint16_t*)(T + nbk * QBB);
    const int dig = (lane & 3) == 3 ? 0 : (lane & 3);  // A row of this lane: digit plane
    const int bq = lane >> 4;                          // this lane's block within a set of four
    const v4i_mf zero = {0, 0, 0, 0};
    for (int b = 0; b < nbk; b += 4) {
        const int bl = min(b + bq, nbk - 1);           // clamped: a block past the chunk adds 0
        const int gb = b0 + bl;
        const int4 a0 = *(const int4*)(xq + (int64_t)gb * 96 + dig * 32);
        const int4 a1 = *(const int4*)(xq + (int64_t)gb * 96 + dig * 32 + 16);
        int w[8];
        if (QT == kQ8_0) {
            const int4 w0 = *(const int4*)(T + b * QBB + lane * 32);
            const int4 w1 = *(const int4*)(T + b * QBB + lane * 32 + 16);
            w[0] = w0.x; w[1] = w0.y; w[2] = w0.z; w[3] = w0.w;
            w[4] = w1.x; w[5] = w1.y; w[6] = w1.z; w[7] = w1.w;
        } else {
            const int4 q = *(const int4*)(T + b * QBB + lane * 16);
            const int qv[4] = {q.x, q.y, q.z, q.w};
            #pragma unroll
            for (int c = 0; c < 4; ++c) {
                w[c] = qv[c] & 0x0F0F0F0F;                             // columns 4c..4c+3 (low nibbles)
                w[4 + c] = (int)(((uint32_t)qv[c] >> 4) & 0x0F0F0F0Fu);  // columns 16+4c.. (high nibbles)
            }
        }
        const float f = (b + bq < nbk ? h2f(sc[b * kTileRows + (lane & 63)]) : 0.f) * xsc[gb];
        const int av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        v4i_mf d0 = zero, d1 = zero;                    // two chains: even and odd column quads
        #pragma unroll
        for (int c = 0; c < 8; c += 2) {
            d0 = __builtin_amdgcn_mfma_i32_4x4x4i8(av[c], w[c], d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_i32_4x4x4i8(av[c + 1], w[c + 1], d1, 0, 0, 0);
        }
        int s0 = d0[0] + d1[0], s1 = d0[1] + d1[1], s2 = d0[2] + d1[2];
        if (QT == kQ4_0) {                              // nibbles n = q + 8: remove 8 x the digit sums
            const int4 Ts = dsum[gb];
            s0 -= 8 * Ts.x;
            s1 -= 8 * Ts.y;
            s2 -= 8 * Ts.z;
        }
        acc = fmaf(f, combine_digits(s0, s1, s2), acc);
    }
}

enum { PH_QKV = 0, PH_ATTN = 1, PH_WO = 2, PH_GU = 3, PH_DOWN = 4, PH_LM = 5 };

// ---- a GEMV phase -------------------------------------------------------------
// The CU's tiles of the phase (row group i, chunk c; t = i * nch + c) go to
// the consumer wavefronts round-robin (t mod 4), so consecutive ring slots
// feed different wavefronts and a group's columns are split among them.  A
// wavefront keeps a partial sum per row (lanes 0..15) for the group it is
// on, and stores it in an LDS buffer when it leaves the group; the
// wavefront that takes the group's last chunk adds the partials in
// wavefront order (fixed, so results are reproducible) and runs the
// epilogue for the group's 16 rows.
struct GroupCtx {
    int gbase;        // cumulative row-group index of the phase's first group (buffer ownership)
};

// lanes l, l+16, l+32, l+48 hold partial sums of row l mod 16 (four input blocks)
__device__ __forceinline__ float row_sum(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

__device__ __forceinline__ bool part_wait(Cons& cs, const int* p, int want_ge) {
    if (lds_get(p) >= want_ge) return true;
    int spins = 0;
    while (lds_get(p) < want_ge) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLds || lds_get(&cs.C->abort)) return cs.fail();
    }
    return true;
}

// store this wavefront's partial of row group gi (cumulative index) in its buffer
__device__ __forceinline__ bool part_store(Cons& cs, int gi, float acc) {
    StepCtl* C = cs.C;
    const int s = gi % kPartBufs;
    if (!part_wait(cs, &C->pdone[s], gi - kPartBufs)) return false;   // the buffer's previous group is finished
    if (cs.lane < kTileRows) C->part[s][cs.cw][cs.lane] = acc;
    drain_lds();
    if (cs.lane == 0) __hip_atomic_fetch_add(&C->pcnt[s], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return true;
}

template <int QT>
__device__ void gemv_phase(Cons& cs, int type, int l, const PhaseMat& pm, int kbase, int gbase, float rs, int p,
                           float* logits, float& best_v, int& best_i) {
    const StepArgs* __restrict__ a = cs.a;
    constexpr int NBK = TileNbk<QT>::value;
    StepCtl* C = cs.C;
    const int G = gridDim.x, cu = blockIdx.x;
    const int nb = pm.g.K >> 5;
    const int8_t* xq = (const int8_t*)cs.xr;
    const float* xsc = (const float*)(xq + (int64_t)nb * 96);
    const int4* dsum = (const int4*)(xsc + ((nb + 3) & ~3));
    const int ngm = my_groups(pm.g.ng, cu, G), nch = pm.g.nch;
    const int nt = ngm * nch;
    const int N = pm.g.N;
    const int lane = cs.lane, j = lane & 15;
    int cur = -1;              // row group this wavefront holds a partial for
    float acc = 0.f;
    for (int t = cs.cw; t < nt; t += kNC) {
        const int i = t / nch, c = t - i * nch;
        if (i != cur) {
            if (cur >= 0 && !part_store(cs, gbase + cur, row_sum(acc))) return;
            cur = i;
            acc = 0.f;
        }
        const int row = (cu + G * i) * kTileRows + j;     // lanes 0..15: this lane's row
        const bool live = lane < kTileRows && row < N;
        const bool last = c == nch - 1;
        float xold = 0.f;
        if (last && (type == PH_WO || type == PH_DOWN) && live)
            xold = ldc(a->x + row);                       // requested before the tile: the round trip overlaps it
        const int k = kbase + t;
        const uint64_t t0 = a->trace ? __builtin_amdgcn_s_memtime() : 0;
        if (!cs.wait_tile(k)) return;
        const uint64_t t1 = a->trace ? __builtin_amdgcn_s_memtime() : 0;
        const uint8_t* T = cs.ring + (int64_t)(k % a->ring_slots) * kStepSlotBytes;
        tile_mfma<QT>(T, last ? pm.g.nbk_last : NBK, c * NBK, xq, xsc, dsum, lane, acc);
        cs.release_tile(k);
        if (a->trace) {
            const uint64_t t2 = __builtin_amdgcn_s_memtime();
            cs.t_wait += t1 - t0;
            cs.t_comp += t2 - t1;
            cs.n_tiles += 1;
        }
        if (!last) continue;

        // finish row group i: every wavefront that took one of its chunks has stored a partial
        const int gi = gbase + i, s = gi % kPartBufs;
        if (!part_store(cs, gi, row_sum(acc))) return;
        cur = -1;
        const int np = nch < kNC ? nch : kNC;             // wavefronts that took a chunk of the group
        if (!part_wait(cs, &C->pcnt[s], np)) return;
        float y = 0.f;
        #pragma unroll
        for (int w = 0; w < kNC; ++w) {
            // wavefront w took a chunk iff some c' < nch has (i * nch + c') mod kNC == w
            const bool took = nch >= kNC || ((w - i * nch) % kNC + kNC) % kNC < nch;
            if (took && lane < kTileRows) y += C->part[s][w][lane];
        }
        drain_lds();
        if (lane == 0) {
            lds_put(&C->pcnt[s], 0);
            lds_put(&C->pdone[s], gi);
        }
        y *= rs;
        const float y1 = __shfl_down(y, 1, 64);          // the odd row of an (even, odd) pair
        if (type == PH_QKV) {
            if (live && (j & 1) == 0) {
                const int hd = a->hd, qrows = a->nq * hd, kvrows = a->nkv * hd;
                __half* kc = a->kcache + (int64_t)l * a->kv_layer;
                __half* vc = a->vcache + (int64_t)l * a->kv_layer;
                if (row < qrows + kvrows) {
                    // RoPE on (2i, 2i+1) of the head: angle p * theta^(-2i/hd)
                    const int rr = row < qrows ? row : row - qrows;
                    const int pi = (rr % hd) >> 1;
                    const float cs_ = ldgf(a->rope_cos + (int64_t)p * (hd >> 1) + pi);
                    const float sn = ldgf(a->rope_sin + (int64_t)p * (hd >> 1) + pi);
                    const float z0 = y * cs_ - y1 * sn;
                    const float z1 = y * sn + y1 * cs_;
                    if (row < qrows) {
                        stc(a->q + row, z0);
                        stc(a->q + row + 1, z1);
                    } else {
                        const __half2 hv = __floats2half2_rn(z0, z1);
                        stc32(kc + ((int64_t)(rr / hd) * a->max_ctx + p) * hd + (rr % hd), *(const uint32_t*)&hv);
                    }
                } else {
                    const int rr = row - qrows - kvrows;
                    const __half2 hv = __floats2half2_rn(y, y1);
                    stc32(vc + ((int64_t)(rr / hd) * a->max_ctx + p) * hd + (rr % hd), *(const uint32_t*)&hv);
                }
            }
        } else if (type == PH_WO || type == PH_DOWN) {
            if (live) stc(a->x + row, xold + y);
        } else if (type == PH_GU) {
            // row 2i = gate i, row 2i+1 = up i: h_i = silu(gate) * up
            if (live && (j & 1) == 0) stc(a->h + (row >> 1), y / (1.0f + __expf(-y)) * y1);
        } else {   // PH_LM
            if (live) {
                if (logits) *gp(logits + row) = y;
                better(best_v, best_i, y, row);
            }
        }
    }
    if (cur >= 0) part_store(cs, gbase + cur, row_sum(acc));
}

// ---- attention: items (KV head, 64-position chunk) over the CUs --------------
template <int HD>
__device__ bool attention(Cons& cs, int l, int p) {
    const StepArgs* __restrict__ a = cs.a;
    constexpr int CH = kAttnCh;
    constexpr int KP = HD + 8;
    constexpr int PCS = CH * HD / 8 / kCT;     // 16-byte pieces per thread per tile
    static_assert(PCS * kCT * 8 == CH * HD, "tile pieces");
    static_assert(4 * kMaxG * HD * 4 <= CH * KP * 2, "PV partials fit over the K tile");
    __half(*Ks)[KP] = (__half(*)[KP])cs.xr;
    __half(*Vs)[HD] = (__half(*)[HD])(cs.xr + CH * KP * 2);
    float(*Qs)[HD] = (float(*)[HD])(cs.xr + CH * KP * 2 + CH * HD * 2);
    float(*Ps)[CH] = (float(*)[CH])((uint8_t*)Qs + kMaxG * HD * 4);
    float* Ms = (float*)((uint8_t*)Ps + kMaxG * CH * 4);
    float* Ls = Ms + kMaxG;
    float(*Os)[kMaxG * HD] = (float(*)[kMaxG * HD])cs.xr;   // reuses the K tile
    const int G = gridDim.x, cu = blockIdx.x;
    const int ct = cs.ct, lane = cs.lane, wave = cs.cw;
    const int GQ = a->nq / a->nkv;
    const int n_ctx = p + 1, n_act = (n_ctx + CH - 1) / CH;
    const int64_t stride = HD + 2;
    const __half* Kl = a->kcache + (int64_t)l * a->kv_layer;
    const __half* Vl = a->vcache + (int64_t)l * a->kv_layer;
    for (int item = cu; item < a->nkv * n_act; item += G) {
        const int g = item / n_act, chunk = item - g * n_act;
        const int t0 = chunk * CH, nt = min(CH, n_ctx - t0);
        const __half* Kg = Kl + (int64_t)g * a->max_ctx * HD;
        const __half* Vg = Vl + (int64_t)g * a->max_ctx * HD;
        uint4 kr[PCS], vr[PCS];
        #pragma unroll
        for (int u = 0; u < PCS; ++u) {
            const int c = ct + u * kCT;
            const int t = min(t0 + c / (HD / 8), a->max_ctx - 1), d8 = (c % (HD / 8)) * 8;
            const __half* kp = Kg + (int64_t)t * HD + d8;
            const __half* vp = Vg + (int64_t)t * HD + d8;
            if (t == p) {          // the row this step appended: device-coherent reads
                const uint64_t k0 = ldc64(kp), k1 = ldc64(kp + 4), v0 = ldc64(vp), v1 = ldc64(vp + 4);
                kr[u] = make_uint4((uint32_t)k0, (uint32_t)(k0 >> 32), (uint32_t)k1, (uint32_t)(k1 >> 32));
                vr[u] = make_uint4((uint32_t)v0, (uint32_t)(v0 >> 32), (uint32_t)v1, (uint32_t)(v1 >> 32));
            } else {
                const int4 k4 = ldg16(kp), v4 = ldg16(vp);
                kr[u] = make_uint4((uint32_t)k4.x, (uint32_t)k4.y, (uint32_t)k4.z, (uint32_t)k4.w);
                vr[u] = make_uint4((uint32_t)v4.x, (uint32_t)v4.y, (uint32_t)v4.z, (uint32_t)v4.w);
            }
        }
        const float* qg = a->q + (int64_t)g * GQ * HD;
        constexpr int QPT = kMaxG * HD / kCT;      // q values per thread (upper bound)
        float qv[QPT];
        #pragma unroll
        for (int u = 0; u < QPT; ++u) qv[u] = ldc(qg + min(ct + u * kCT, GQ * HD - 1));
        #pragma unroll
        for (int u = 0; u < PCS; ++u) {
            const int c = ct + u * kCT;
            const int t = c / (HD / 8), d8 = (c % (HD / 8)) * 8;
            *(uint4*)&Ks[t][d8] = kr[u];
            *(uint4*)&Vs[t][d8] = vr[u];
        }
        #pragma unroll
        for (int u = 0; u < QPT; ++u) {
            const int i = ct + u * kCT;
            if (i < GQ * HD) Qs[i / HD][i % HD] = qv[u];
        }
        if (!cs.sync(false)) return false;

        // scores: a wavefront per query head, a lane per key; causal mask
        for (int j = wave; j < GQ; j += kNC) {
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
                sc = (acc0 + acc1) * a->scale;
            }
            const float m = wave_max(sc);
            const float pv = lane < nt ? __expf(sc - m) : 0.f;
            const float lv = wave_sum(pv);
            Ps[j][lane] = pv;
            if (lane == 0) { Ms[j] = m; Ls[j] = lv; }
        }
        if (!cs.sync(false)) return false;

        // o = sum_t p_t v_t: thread (head j, 8 dims, quarter w of the keys)
        constexpr int D8 = HD / 8;
        for (int idx = ct; idx < GQ * D8 * kNC; idx += kCT) {
            const int w = idx / (GQ * D8), r = idx % (GQ * D8);
            const int j = r / D8, d8 = (r % D8) * 8;
            float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            const int tb = w * (CH / kNC), te = min(tb + CH / kNC, nt);
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
        if (!cs.sync(false)) return false;

        float* part = a->attn_part;
        float* out = a->o + (int64_t)g * GQ * HD;
        if (n_act == 1) {
            for (int i = ct; i < GQ * HD; i += kCT) {
                float v = Os[0][i];
                #pragma unroll
                for (int w = 1; w < kNC; ++w) v += Os[w][i];
                stc(out + i, v / Ls[i / HD]);
            }
        } else {
            for (int i = ct; i < GQ * HD; i += kCT) {
                float v = Os[0][i];
                #pragma unroll
                for (int w = 1; w < kNC; ++w) v += Os[w][i];
                const int j = i / HD, d = i % HD;
                float* ph = part + ((int64_t)(g * GQ + j) * a->max_chunks + chunk) * stride;
                stc(ph + d, v);
                if (d == 0) {
                    stc(ph + HD, Ms[j]);
                    stc(ph + HD + 1, Ls[j]);
                }
            }
            if (!cs.sync(true)) return false;          // partials complete before the count
            if (wave == 0 && lane == 0) {
                const uint32_t old = addc32(a->attn_cnt + g, 1u);
                lds_put(&cs.C->flag, old == (uint32_t)(n_act - 1) ? 1 : 0);
            }
            if (!cs.sync(false)) return false;
            if (lds_get(&cs.C->flag)) {
                // the last chunk of KV head g merges all chunks (log-sum-exp)
                for (int idx = ct; idx < GQ * HD; idx += kCT) {
                    const int j = idx / HD, d = idx % HD;
                    const float* ph = part + (int64_t)(g * GQ + j) * a->max_chunks * stride;
                    float M = -FLT_MAX, L = 0.f, O = 0.f;
                    constexpr int B = 8;
                    for (int base = 0; base < n_act; base += B) {
                        float mv[B], lv[B], ov[B];
                        #pragma unroll
                        for (int u = 0; u < B; ++u) {
                            const int c = min(base + u, n_act - 1);
                            mv[u] = ldc(ph + c * stride + HD);
                            lv[u] = ldc(ph + c * stride + HD + 1);
                            ov[u] = ldc(ph + c * stride + d);
                        }
                        float bm = M;
                        #pragma unroll
                        for (int u = 0; u < B; ++u)
                            if (base + u < n_act) bm = fmaxf(bm, mv[u]);
                        const float r = __expf(M - bm);
                        L *= r;
                        O *= r;
                        #pragma unroll
                        for (int u = 0; u < B; ++u)
                            if (base + u < n_act) {
                                const float e = __expf(mv[u] - bm);
                                L = fmaf(lv[u], e, L);
                                O = fmaf(ov[u], e, O);
                            }
                        M = bm;
                    }
                    stc(out + idx, O / L);
                }
                if (wave == 0 && lane == 0) stc32(a->attn_cnt + g, 0u);
            }
        }
        if (!cs.sync(false)) return false;             // LDS free for the next item
    }
    return true;
}

// ---- the consumer side of the step ------------------------------------------
template <int QT, int HD>
__device__ void consumer(const StepArgs* __restrict__ a, const int* tokens, float* logits, int* argmax_out,
                         uint8_t* ring, uint8_t* xr, StepCtl* C, int cw, int lane) {
    Cons cs(a, ring, xr, C, cw, lane);
    cs.epoch = ldc32(a->epoch);
    const int G = gridDim.x, cu = blockIdx.x;
    const int p = (int)ldc32(a->pos);
    int tok = *gp(tokens);
    if (tok < 0 || tok >= a->V) tok = 0;
    float best_v = -FLT_MAX;
    int best_i = INT_MAX;
    int kbase = 0, gbase = 0, wp = 0;
    const int n_phase = 5 * a->L + 1;
    for (int ph = 0; ph < n_phase; ++ph) {
        const int l = ph / 5;
        const int type = ph == 5 * a->L ? PH_LM : ph % 5;
        if (cw == 0 && lane == 0) trace_at(a, ph, 0);
        if (type == PH_ATTN) {
            if (!attention<HD>(cs, l, p)) break;
        } else {
            const PhaseMat pm = phase_mat(a, wp);
            const float* src = a->x;
            const uint16_t* emb = nullptr;
            const float* gain = nullptr;
            float* x_out = nullptr;
            if (type == PH_QKV) {
                gain = a->norms + (int64_t)l * 2 * a->H;
                if (l == 0) {
                    emb = a->embd + (int64_t)tok * a->H;
                    if (cu == 0) x_out = a->x;
                }
            } else if (type == PH_WO) {
                src = a->o;
            } else if (type == PH_GU) {
                gain = a->norms + ((int64_t)l * 2 + 1) * a->H;
            } else if (type == PH_DOWN) {
                src = a->h;
            } else {
                gain = a->out_norm;
            }
            const float rs = stage_input<QT>(cs, src, emb, gain, pm.g.K, x_out);
            if (!cs.ok) break;
            if (cw == 0 && lane == 0) trace_at(a, ph, 1);
            gemv_phase<QT>(cs, type, l, pm, kbase, gbase, rs, p, logits, best_v, best_i);
            if (!cs.ok) break;
            if (cw == 0 && lane == 0) {
                trace_at(a, ph, 2);
                if (a->trace) {
                    uint64_t* tw = a->trace + ((int64_t)blockIdx.x * (5 * a->L + 1) + ph) * kTraceWords;
                    *gp(tw + 5) = cs.t_wait;
                    *gp(tw + 6) = cs.t_comp;
                    *gp(tw + 7) = cs.n_tiles;
                }
            }
            cs.t_wait = cs.t_comp = cs.n_tiles = 0;
            kbase += my_groups(pm.g.ng, cu, G) * pm.g.nch;
            gbase += my_groups(pm.g.ng, cu, G);
            ++wp;
        }
        if (ph + 1 < n_phase && !cs.grid_barrier(ph)) break;
    }

    if (cs.ok) {
        // argmax: lanes -> consumer wavefronts -> this CU's partial -> the last CU reduces
        #pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(best_v, off, 64);
            const int oi = __shfl_xor(best_i, off, 64);
            better(best_v, best_i, ov, oi);
        }
        if (lane == 0) {
            C->bv[cw] = best_v;
            C->bi[cw] = best_i;
        }
        if (cs.sync(true) && cw == 0) {
            float bv = C->bv[0];
            int bi = C->bi[0];
            #pragma unroll
            for (int w = 1; w < kNC; ++w) better(bv, bi, C->bv[w], C->bi[w]);
            uint32_t old = 0;
            if (lane == 0) {
                stc(a->part_val + cu, bv);
                stc32(a->part_idx + cu, (uint32_t)bi);
                drain_vm();
                old = addc32(a->done_cnt, 1u);
            }
            old = __shfl(old, 0, 64);
            if (old == (uint32_t)(G - 1)) {
                float v = -FLT_MAX;
                int vi = INT_MAX;
                for (int i = lane; i < G; i += 64) better(v, vi, ldc(a->part_val + i), (int)ldc32(a->part_idx + i));
                #pragma unroll
                for (int off = 32; off > 0; off >>= 1) {
                    const float ov = __shfl_xor(v, off, 64);
                    const int oi = __shfl_xor(vi, off, 64);
                    better(v, vi, ov, oi);
                }
                if (lane == 0) {
                    *gp(argmax_out) = vi;
                    *gp(a->pos) = p + 1;
                    stc32(a->done_cnt, 0u);
                    stc32(a->epoch, cs.epoch + 1u);
                }
            }
        }
    }
    if (!cs.ok && lane == 0) stc32(a->err, 1u);
}

template <int QT, int HD>
__global__ __launch_bounds__(kStepThreads, 1) void k_step(const StepArgs* __restrict__ a, const int* tokens,
                                                          float* logits, int* argmax_out) {
    extern __shared__ __align__(16) uint8_t lds[];
    uint8_t* ring = lds;
    uint8_t* xr = lds + (int64_t)a->ring_slots * kStepSlotBytes;
    StepCtl* C = (StepCtl*)(xr + a->xbytes);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int i = tid; i < kStepMaxSlots; i += kStepThreads) {
        C->ready[i] = -1;
        C->done[i] = i - a->ring_slots;
    }
    for (int i = tid; i < kPartBufs; i += kStepThreads) {
        C->pcnt[i] = 0;
        C->pdone[i] = i - kPartBufs;
    }
    if (tid == 0) {
        C->csync = 0;
        C->gen = 0;
        C->abort = 0;
        C->flag = 0;
    }
    __syncthreads();
    if (wave < kNP) producer<QT>(a, ring, C, wave, lane);
    else consumer<QT, HD>(a, tokens, logits, argmax_out, ring, xr, C, wave - kNP, lane);
}

template <int QT, int HD>
static hipError_t launch_t(const StepArgs& h, const StepArgs* d, const int* tokens, float* logits, int* argmax_out,
                           int n_cus, hipStream_t st) {
    const size_t lds = (size_t)h.ring_slots * kStepSlotBytes + h.xbytes + kStepCtlBytes;
    (void)hipFuncSetAttribute((const void*)k_step<QT, HD>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL((k_step<QT, HD>), dim3(n_cus), dim3(kStepThreads), lds, st, d, tokens, logits, argmax_out);
    return hipGetLastError();
}

hipError_t launch_step(const StepArgs& h, const StepArgs* d, int qtype, const int* tokens, float* logits,
                       int* argmax_out, int n_cus, hipStream_t st) {
    if (h.ring_slots < 4 || h.ring_slots > kStepMaxSlots) return hipErrorInvalidValue;
    if ((size_t)h.ring_slots * kStepSlotBytes + h.xbytes + kStepCtlBytes > (size_t)kStepLdsMax)
        return hipErrorInvalidValue;
    if (h.hd != 64 && h.hd != 128) return hipErrorInvalidValue;
    if (qtype == kQ8_0)
        return h.hd == 128 ? launch_t<kQ8_0, 128>(h, d, tokens, logits, argmax_out, n_cus, st)
                           : launch_t<kQ8_0, 64>(h, d, tokens, logits, argmax_out, n_cus, st);
    return h.hd == 128 ? launch_t<kQ4_0, 128>(h, d, tokens, logits, argmax_out, n_cus, st)
                       : launch_t<kQ4_0, 64>(h, d, tokens, logits, argmax_out, n_cus, st);
}

}  // namespace lmk
