// lm_step.h - the persistent one-kernel decode step: tile-major weight
// geometry and kernel arguments, shared by the host runtime and the kernel.
#pragma once

#include "lm_internal.h"

namespace lmk {

constexpr int kStepSlotBytes = 9216;   // one LDS ring slot = one weight tile
constexpr int kStepMaxSlots = 16;
constexpr int kTileRows = 16;          // rows per tile (one MFMA operand of weights)
constexpr int kTileRowsFwd = kTileRows;
constexpr int kTileBlocksQ8 = 16;      // 32-column blocks per tile: 16 x 16 x 34 = 8704 bytes
constexpr int kTileBlocksQ4 = 32;      //                            16 x 32 x 18 = 9216 bytes
constexpr int kBarStride = 32 * 10;    // barrier words per phase: a global count and up to 8
                                       // per-XCD counts, each on its own 128-byte line
constexpr int kPartBufs = 16;          // row-group partial-sum buffers (K split among consumers)
constexpr int kStepCtlBytes = 512 + kPartBufs * 4 * kTileRowsFwd * 4;   // LDS control block + partials
constexpr int kStepLdsMax = 163840;    // LDS per workgroup on gfx950

// Tile-major layout of one quantised matrix [N rows][K cols]:
//   rows in groups of 16 (zero rows pad the last group), each group's
//   columns in chunks of NBK blocks; tile (group, chunk) is contiguous:
//     Q8_0: for each block b: for row j = 0..15: the row's 32 quants of the
//           block (512 bytes per block); then the fp16 scales [b][j]
//     Q4_0: for each block b: for row j = 0..15: the row's 16 nibble bytes
//           of the block in GGUF order (byte i: column i low, column i+16
//           high; 256 bytes per block); then the fp16 scales [b][j]
//   a group's chunks follow each other, groups follow each other.  Bytes per
//   weight are exactly the GGUF ones.  Four consecutive blocks of a tile are
//   one matrix-core operand set: lane l of a wavefront reads row l mod 16 of
//   block l / 16 at offset 32 l (Q8_0) or 16 l (Q4_0).
struct TileGeom {
    int N, K;
    int ng;         // row groups
    int nch;        // column chunks
    int nbk_last;   // blocks in the last chunk
    int tfull;      // bytes of a full tile
    int ufull;      // 16-byte units of a full tile
    int ulast;      // 16-byte units of the last chunk's tile
    int64_t gbytes; // bytes of one row group (all its chunks)
};

inline TileGeom tile_geom(int qtype, int N, int K) {
    const int nbk = qtype == kQ8_0 ? kTileBlocksQ8 : kTileBlocksQ4;
    const int bb = qtype == kQ8_0 ? 34 : 18;
    const int nb = K / 32;
    TileGeom g;
    g.N = N;
    g.K = K;
    g.ng = (N + kTileRows - 1) / kTileRows;
    g.nch = (nb + nbk - 1) / nbk;
    g.nbk_last = nb - (g.nch - 1) * nbk;
    g.tfull = (kTileRows * nbk * bb + 15) / 16 * 16;
    const int tlast = (kTileRows * g.nbk_last * bb + 15) / 16 * 16;
    g.ufull = g.tfull / 16;
    g.ulast = tlast / 16;
    g.gbytes = (int64_t)(g.nch - 1) * g.tfull + tlast;
    return g;
}
inline int64_t tile_matrix_bytes(const TileGeom& g) { return (int64_t)g.ng * g.gbytes; }

// LDS bytes of the per-phase input (integer digits of the widest input) or
// of the attention scratch, whichever is larger
inline int step_xbytes(int qtype, int kmax, int hd) {
    const int nb = kmax / 32;
    int digits = nb * 96 + ((nb + 3) & ~3) * 4 + (qtype == kQ4_0 ? nb * 16 : 0);
    const int attn = 64 * (hd + 8) * 2 + 64 * hd * 2 + 8 * hd * 4 + 8 * 64 * 4 + 16 * 4;
    const int x = digits > attn ? digits : attn;
    return (x + 15) / 16 * 16;
}
inline int step_ring_slots(int xbytes) {
    const int n = (kStepLdsMax - xbytes - kStepCtlBytes) / kStepSlotBytes;
    return n > kStepMaxSlots ? kStepMaxSlots : n;
}

struct StepArgs {
    int L, H, F, V, nq, nkv, hd, max_ctx;
    float eps, scale;
    const uint8_t* tiles;      // tile-major layer matrices: layer l at tiles + l * layer_stride
    int64_t layer_stride;
    int64_t mat_off[4];        // QKV, Wo, gate/up (rows interleaved), down within a layer
    const uint8_t* lm_tiles;   // tile-major LM head
    TileGeom geo[5];           // QKV, Wo, gate/up, down, LM head
    const uint16_t* embd;      // fp16 [V][H]
    const float* norms;        // fp32 [L][2][H] (attention, FFN)
    const float* out_norm;     // fp32 [H]
    __half* kcache;            // [L][max_seqs][nkv][max_ctx][hd]; sequence 0 is decoded
    __half* vcache;
    int64_t kv_layer;          // elements per layer
    const float* rope_cos;     // [max_ctx][hd/2]
    const float* rope_sin;
    int* pos;                  // [1] position; advanced by one at the end
    float *x, *q, *o, *h;      // activations exchanged between CUs
    float* attn_part;          // [nq][max_chunks][hd + 2]
    uint32_t* attn_cnt;        // [nkv], zero between launches
    int max_chunks;
    float* part_val;           // [grid] argmax partials
    int* part_idx;
    uint32_t* done_cnt;        // [1], zero between launches
    uint32_t* bar;             // [phases][kBarStride], counts grow by one round per launch
    uint32_t* epoch;           // [1] completed launches (barrier round)
    int* err;                  // [1] set on a timed-out wait
    int ring_slots;
    int xbytes;
    uint64_t* trace;           // nullptr, or [grid][5L+1][kTraceWords] timestamps (debug)
};
constexpr int kTraceWords = 8;     // per (CU, phase): see lm_debug_step_trace

// grid = one workgroup per CU (all resident), 512 threads, dynamic LDS.
// h: the arguments on the host (launch geometry); d: the same arguments in
// device memory (what the kernel reads); tokens [1], logits [V] or nullptr,
// argmax_out [1]: per-call device buffers.
hipError_t launch_step(const StepArgs& h, const StepArgs* d, int qtype, const int* tokens, float* logits,
                       int* argmax_out, int n_cus, hipStream_t st);
inline int64_t step_bar_words(int n_layers) { return (int64_t)(5 * n_layers + 1) * kBarStride; }

}  // namespace lmk
