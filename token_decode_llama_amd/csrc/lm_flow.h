// lm_flow.h - the dataflow decode step: every layer of one batch-1 step in a
// single launch, workgroups ordered by dependency (see lm_flow.hip).
#pragma once

#include "lm_internal.h"

namespace lmk {

constexpr int kFlowOps = 5;    // per layer: QKV, attention, Wo, gate/up, down
constexpr int kFlowSub = 16;   // partial completion counters per phase
constexpr int kFlowLine = 32;  // words per counter (one 128-byte line each)
inline int64_t flow_ctl_words(int n_layers) {
    return (int64_t)n_layers * kFlowOps * (kFlowSub + 1) * kFlowLine + 2 * kFlowLine;
}

// one quantised matrix inside a layer blob (layout of QMat)
struct FlowMat {
    int64_t q_off, sc_off;
    int N, K;
};

struct FlowArgs {
    int L, H, F, nq, nkv, hd, max_ctx, max_chunks;
    float eps, scale;
    const uint8_t* blobs;      // layer l at blobs + l * blob_stride
    int64_t blob_stride;
    FlowMat mat[4];            // QKV, Wo, gate/up (rows interleaved), down
    const float* norms;        // fp32 [L][2][H] (attention, FFN)
    __half* kcache;            // [L][max_seqs][nkv][max_ctx][hd]; sequence 0 is decoded
    __half* vcache;
    int64_t kv_layer;          // elements per layer
    const int* pos;            // [1] current position (advanced by the LM head afterwards)
    const float* rope_cos;     // [max_ctx][hd/2]
    const float* rope_sin;
    float *x, *q, *o, *h;      // activations exchanged between workgroups
    float* attn_part;          // [nq][max_chunks][hd + 2]
    int* attn_cnt;             // [nkv][attn_cnt_lines][kCntStride] (chunk_arrive), zero between uses
    uint32_t* done;            // [L * kFlowOps][kFlowSub + 1][kFlowLine] phase counters, one per
                               // 128-byte line: kFlowSub partial counts (workgroup index mod
                               // kFlowSub) and the count of complete partials; all grow by their
                               // launch total every launch
    uint32_t* epoch;           // [1] completed launches
    uint32_t* err;             // [1] set when a wait timed out
    int wg[kFlowOps];          // workgroups per phase
    int wg_off[kFlowOps + 1];  // prefix sums; wg_off[kFlowOps] = workgroups per layer
    uint64_t* trace;           // nullptr, or [rows][kFlowTraceWords] (debug): start, wait
                               // passed, work done (100 MHz clock), hardware ids; a row per
                               // workgroup (dataflow) or per (phase, workgroup) (resident)
    int resident;              // 1: every workgroup stays for every phase (grid = wg[0])
};
constexpr int kFlowTraceWords = 4;

// true when the dataflow step supports this shape (Q8_0 / Q4_0, head_dim 128,
// at most 8 query heads per KV head, H and F at least 2048 and multiples of 32)
bool flow_supported(int qtype, int H, int F, int hd, int nq, int nkv);
// dynamic LDS bytes of a workgroup
int flow_lds_bytes(int qtype, int H, int F, int hd);
// workgroups per phase for this shape on `n_cus` compute units (host; queries
// the kernel's occupancy, so the device must be current)
void flow_plan(FlowArgs& a, int qtype, int n_cus);
// one launch: all L layers (the embedding before and the LM head after are
// separate launches).  Asynchronous on `st`.
hipError_t launch_flow(const FlowArgs& a, int qtype, hipStream_t st);

}  // namespace lmk
