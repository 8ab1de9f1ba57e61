// lm_internal.h - shared declarations between the host runtime and the
// gfx950 kernels of the decode step (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace lmk {

constexpr int kQ4_0 = 2;
constexpr int kQ8_0 = 8;
constexpr int kQ4_K = 12;   // GGUF K formats: 256-weight super-blocks (batch-1 GEMV only)
constexpr int kQ5_K = 13;
constexpr int kQ6_K = 14;
constexpr bool is_kquant(int qtype) { return qtype == kQ4_K || qtype == kQ5_K || qtype == kQ6_K; }
constexpr int kAttnChunk = 64;     // KV positions per attention workgroup
constexpr int kCntStride = 32;     // ints per attention chunk counter: one 128-byte line each, so
                                   // that different counters do not serialise each other's atomics
constexpr int kCntGroup = 16;      // chunks per first-level counter (atomics on one line serialise)
// counter lines per (sequence, KV head): the count of complete groups, then one per group
constexpr int attn_cnt_lines(int max_chunks) { return 1 + (max_chunks + kCntGroup - 1) / kCntGroup; }

// Device layout of one quantised matrix [N rows][K cols], nb = K/32 blocks/row,
// nsb = K/256 super-blocks/row (K formats).  Quants and scales sit in two
// planes, row-major, so that a row range of a matrix is a contiguous slice:
//   Q8_0: quants, each row = [first 16 bytes of every block]
//         [last 16 bytes of every block] (int8), so a wavefront reading
//         block b of consecutive lanes makes fully coalesced 16-byte loads;
//         scales: fp16 [N/2][nb][2], the two rows of a row pair interleaved
//         (one 32-bit load gives both rows' scale of a block; kScPairs),
//         else fp16 [N][nb];
//   Q4_0: quants, each row = nb x 16 nibble bytes in GGUF order
//         (byte j: element j low nibble, element j+16 high nibble);
//         scales: fp16 [N/2][nb][2] as Q8_0;
//   Q4_K: quants, each row = nb x 16 bytes, the 32-weight sub-blocks
//         regrouped into the Q4_0 nibble order; scales: the super-blocks'
//         16-byte headers as stored (fp16 d, fp16 dmin, 12 bytes of packed
//         6-bit scale/min pairs) [N][nsb][16];
//   Q5_K: as Q4_K, each quant row followed by nb x 4 bytes of fifth bits: the
//         32-bit word of a block holds element 4u+k's bit at bit 8k + u and
//         element 16+4u+k's at bit 8k + 4 + u (u, k < 4);
//   Q6_K: quants, each row = nb x 16 bytes of low nibbles (Q4_0 order), then
//         nb x 8 bytes of 2-bit high parts: words h0 (elements 0..15) and h1
//         (16..31) of a block hold element 4u+k's (u, k < 4) two bits at bit
//         8k + 2u; scales, each row = nb x 2 int8 (the two 16-weight
//         sub-block scales of each block), then nsb x fp16 d.
// Every layout holds exactly the GGUF bytes of the matrix, regrouped.
struct QMat {
    const uint8_t* q;
    const uint16_t* sc;
    const uint16_t* sct;   // scales again for the matrix-core GEMV: per 16-row tile, 4-block group,
                           // row, block (sct_bytes in lm_runtime.cpp; models that decode several
                           // sequences at once)
    const uint8_t* qf;     // quants again, as matrix-core A fragments (same models; below)
    int N, K;
};

// Matrix-core fragment copy of the quants: per 16-row tile t and group of
// qfrag_blocks consecutive blocks, 64 lane slices of 16 bytes; lane l = 16g + j
// holds row j of the tile, columns 8g..8g+7 of each block of the group:
//   Q8_0: 2 blocks x 8 int8;  Q4_0: 4 blocks x 4 bytes, byte i = nibble of
//   column 8g+i (low) | nibble of column 8g+4+i (high).
// Offset of (t, group, lane) = ((t * groups + group) * 64 + l) * 16.
inline int qfrag_blocks(int qtype) { return qtype == kQ8_0 ? 2 : 4; }
inline int64_t qfrag_bytes(int qtype, int64_t N, int64_t K) {
    const int64_t nb = K / 32, per = qfrag_blocks(qtype);
    return (N + 15) / 16 * ((nb + per - 1) / per) * 1024;
}

constexpr int64_t qmat_qbytes(int qtype, int64_t N, int64_t K) {
    if (qtype == kQ8_0) return N * K;
    if (qtype == kQ6_K) return N * (K / 2 + K / 4);
    if (qtype == kQ5_K) return N * (K / 2 + K / 8);
    return N * K / 2;
}
// bytes of one row of the scale plane
constexpr int64_t qmat_srow(int qtype, int64_t K) {
    if (qtype == kQ4_K || qtype == kQ5_K) return K / 256 * 16;
    if (qtype == kQ6_K) return K / 32 * 2 + K / 256 * 2;
    return K / 32 * 2;
}
constexpr int64_t qmat_sbytes(int qtype, int64_t N, int64_t K) { return N * qmat_srow(qtype, K); }
// bytes of one GGUF row of K weights
inline int64_t gguf_row_bytes(int qtype, int64_t K) {
    switch (qtype) {
        case kQ8_0: return K / 32 * 34;
        case kQ4_0: return K / 32 * 18;
        case kQ4_K: return K / 256 * 144;
        case kQ5_K: return K / 256 * 176;
        default: return K / 256 * 210;
    }
}

enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

// Q8_0 / Q4_0 scale plane: 1 = the two rows of a row pair interleaved per
// block (one 32-bit load per block for both rows), 0 = row-major [N][nb].
#ifndef LMK_SC_PAIRS
#define LMK_SC_PAIRS 1
#endif
constexpr bool kScPairs = LMK_SC_PAIRS != 0;

struct GemvArgs {
    QMat w;
    int qtype;
    const float* xin;      // [n_seq][x_stride] input activations
    int x_stride;
    const float* norm_g;   // RMSNorm gain applied to xin first, or nullptr
    float eps;
    // epilogue outputs
    float* out;            // QKV: q [n_seq][nq*hd]; RESID: x [n_seq][N] (+=);
                           // SWIGLU: h [n_seq][N/2]; LOGITS: logits [n_seq][N] or nullptr
    int out_stride;
    // QKV epilogue
    int q_rows, kv_rows, head_dim, max_ctx;
    __half* kcache;        // layer base [max_seqs][nkv][max_ctx][hd]
    __half* vcache;
    int64_t kv_seq_stride; // elements per sequence in one layer's cache
    const int* pos;        // [n_seq] current position of each sequence
    const float* rope_cos; // [max_ctx][hd/2]
    const float* rope_sin;
    // LOGITS epilogue: per-workgroup (max, index) partials and the final argmax
    float* part_val;       // [n_seq][gridDim.x]
    int* part_idx;
    int* counter;          // [n_seq], zero between launches
    int* argmax_out;       // [n_seq]
    int* pos_inc;          // [n_seq] positions advanced by one after the argmax
    // several sequences at once (MFMA path)
    int n_seq;
    uint8_t* xfrag;        // activation digits, scales and digit sums (xfrag_bytes; lm_kernels.hip)
    int xfrag_ready;       // wide-input GEMV: xfrag already holds this input's digits (written by
                           // the gate/up kernel's epilogue), so no digit kernel runs first
};

struct AttnArgs {
    const float* q;        // [n_seq][nq*hd], rotated
    const __half* kcache;  // layer base [max_seqs][nkv][max_ctx][hd]
    const __half* vcache;
    int64_t kv_seq_stride;
    const int* pos;
    int nq, nkv, hd, max_ctx, max_chunks;
    float scale;           // 1/sqrt(hd)
    int grid_chunks;       // chunks the grid covers (<= max_chunks; >= every sequence's context)
    int tiles;             // kAttnChunk-position tiles per workgroup (attn_tiles), >= 1
    float* part;           // [n_seq][nq][max_chunks][hd + 2] partial o, m, l (one record per workgroup)
    int* counter;          // [n_seq][nkv][attn_cnt_lines][kCntStride] chunk counts (first int of
                           // each line, see chunk_arrive), zero between launches
    float* out;            // [n_seq][nq*hd]
};

// launchers (lm_kernels.hip); all asynchronous on `st`
hipError_t launch_embed(const uint16_t* tok_embd, const int* tokens, int vocab, int hidden,
                        float* x, int n_seq, hipStream_t st);
hipError_t launch_gemv(const GemvArgs& a, int epi, int n_seq, int max_blocks, hipStream_t st);
// 2..4 sequences: the matrix-core GEMV (its activation digits computed in each
// workgroup's prologue, or for wide inputs by a digit kernel into a.xfrag first)
hipError_t launch_gemv_batched(const GemvArgs& a, int epi, int n_seq, int max_blocks, hipStream_t st);
// The several-sequence gate/up GEMV of an FFN of width ffn writes the digits
// of its output h into a.xfrag itself (the down projection then sets
// xfrag_ready) when h is too wide for the down GEMV's own prologue.
bool gateup_writes_digits(int64_t ffn);
// Activation operands of the several-sequence GEMV for nb = K/32 blocks:
// digits uint2 [nb][4 column groups][16 rows 4s+d], then activation scales
// fp32 [nb][4 sequences], then digit sums int4 [nb][4 sequences].
inline int64_t xfrag_bytes(int64_t K) { return K / 32 * (512 + 16 + 64); }
int attn_tiles(int n_seq, int nkv, int max_chunks, int hd);
hipError_t launch_attention(const AttnArgs& a, int n_seq, hipStream_t st);
hipError_t launch_dequant(const QMat& w, int qtype, int row0, int n_rows, float* out,
                          hipStream_t st);
hipError_t launch_read_bw(const void* buf, int64_t n_bytes, float* sink, hipStream_t st);
// The allocation-free step's scratch (lm_kernels.hip): a fixed device array of
// kNoAllocScratchBytes per device, its address looked up once per device.
constexpr int64_t kNoAllocScratchBytes = 32ll << 20;
hipError_t noalloc_scratch(int device, uint8_t** ptr);
// p[0..n) = 0 with a kernel (a graph under capture gets a kernel node, not a memset node)
hipError_t launch_zero(void* p, int64_t n_bytes, hipStream_t st);
// acc[0] += cosine similarity of xin and x ([n_seq][H] each) summed over the sequences, acc[1] += n_seq
hipError_t launch_layer_cos(const float* xin, const float* x, int H, int n_seq, double* acc, hipStream_t st);

}  // namespace lmk
