// lm_runtime.cpp - host runtime behind the C ABI in include/lmdecode.h.
//
// One model = one HIP stream (plus a copy stream for weight streaming).  All
// device memory is allocated in lm_model_create, so a decode step allocates
// nothing.  Weight matrices are repacked at load into the layout the GEMV
// kernels read (lm_internal.h); one layer's four matrices form one
// contiguous "layer blob", which is also the unit the streaming mode copies.
//
// Streaming mode follows the double-buffered layer pipeline of the C/CUDA
// Llama engine page (rskf.cn/news/15116, sections 2.3, 3.3 and 4.2: compute
// layer n from one buffer while layer n+1 loads into the other, then swap)
// and the pinned host region + two device ping-pong buffers + two streams +
// per-layer events of "3 Agents. 3 LLMs. 1 Aging GPU" (section on loading
// only the layers you need).  Both ordering edges are explicit events: a
// layer's compute waits for its copy, and the copy that overwrites a buffer
// waits for the compute that last read it.
#include "lm_internal.h"

#include "../../include/lmdecode.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <unistd.h>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

using namespace lmk;

namespace {

thread_local std::string g_create_error;
std::atomic<long> g_alloc_count{0};
std::atomic<long> g_fail_at{0};

constexpr int64_t kAlign = 256;
inline int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Matrices of one layer blob, in order.
enum { M_QKV = 0, M_WO = 1, M_GU = 2, M_DOWN = 3, M_COUNT = 4 };

struct MatOff {
    int64_t q, sc;   // byte offsets within the blob
    int64_t sct;     // transposed scales [ceil(N/16)][nb][16], or -1 (single-sequence models)
    int64_t qf;      // matrix-core fragment copy of the quants (lm_internal.h), or -1
    int N, K;
};

// bytes of a tile-transposed scale plane
// scales for the matrix-core GEMV: [N/16 tiles][ceil(nb/4) groups][16 rows][4 blocks] fp16
// (zero past the last row and block): a row's scales of one 4-block stage are 8 contiguous bytes
inline int64_t sct_bytes(int64_t N, int64_t K) { return (N + 15) / 16 * ((K / 32 + 3) / 4) * 64 * 2; }

template <class F>
void parallel_rows(int64_t n, F&& fn) {
    unsigned nt = std::min<unsigned>(std::max(1u, std::thread::hardware_concurrency()), 16u);
    if (n < 64 || nt <= 1) { fn(0, n); return; }
    std::vector<std::thread> th;
    const int64_t per = (n + nt - 1) / nt;
    for (unsigned t = 0; t < nt; ++t) {
        const int64_t a = t * per, b = std::min(n, a + per);
        if (a >= b) break;
        th.emplace_back([&fn, a, b] { fn(a, b); });
    }
    for (auto& t : th) t.join();
}

// GGUF row -> device layout row (quants + scales; lm_internal.h).  The K
// formats (GGUF's published layout; the C/CUDA Llama engine page, section 1,
// names them): Q4_K super-block = fp16 d, fp16 dmin, 12 bytes of 6-bit
// scale/min pairs, 128 bytes whose 32-byte group g holds sub-block 2g in the
// low nibbles and 2g+1 in the high ones; Q6_K super-block = 128 bytes of low
// nibbles (element 128h + 32t + l at byte 64h + 32(t%2) + l, high nibble when
// t >= 2), 64 bytes of 2-bit high parts (bits 2t, 2t+1 of byte 32h + l),
// 16 int8 sub-block scales, fp16 d.
// Q8_0 / Q4_0 block scales are interleaved per row pair when kScPairs (row
// 2i's scale of block b, then row 2i+1's): the caller points dsc at this
// row's first one, and consecutive blocks are 4 bytes apart (else 2).
void repack_row(int qtype, const uint8_t* src, int K, uint8_t* dq, uint8_t* dsc) {
    const int nb = K / 32;
    if (qtype == kQ8_0) {
        for (int b = 0; b < nb; ++b) {
            const uint8_t* blk = src + (int64_t)b * 34;
            std::memcpy(dsc + (kScPairs ? 4 : 2) * b, blk, 2);
            std::memcpy(dq + (int64_t)b * 16, blk + 2, 16);
            std::memcpy(dq + (int64_t)nb * 16 + (int64_t)b * 16, blk + 18, 16);
        }
    } else if (qtype == kQ4_0) {
        for (int b = 0; b < nb; ++b) {
            const uint8_t* blk = src + (int64_t)b * 18;
            std::memcpy(dsc + (kScPairs ? 4 : 2) * b, blk, 2);
            std::memcpy(dq + (int64_t)b * 16, blk + 2, 16);
        }
    } else if (qtype == kQ4_K || qtype == kQ5_K) {
        // Q5_K: the Q4_K header, 32 bytes of fifth bits (bit j of byte l: element 32j + l), the nibbles
        const bool five = qtype == kQ5_K;
        const int bytes = five ? 176 : 144, nib = five ? 48 : 16;
        if (five) std::memset(dq + (int64_t)nb * 16, 0, (size_t)nb * 4);
        for (int sb = 0; sb < K / 256; ++sb) {
            const uint8_t* blk = src + (int64_t)sb * bytes;
            std::memcpy(dsc + 16 * sb, blk, 16);
            for (int j = 0; five && j < 8; ++j) {
                uint8_t* h = dq + (int64_t)nb * 16 + (int64_t)(8 * sb + j) * 4;
                for (int i = 0; i < 32; ++i) {
                    const int bit = (blk[16 + i] >> j) & 1, ii = i & 15;
                    h[(ii & 3)] |= (uint8_t)(bit << ((ii >> 2) + (i < 16 ? 0 : 4)));
                }
            }
            for (int j = 0; j < 8; ++j) {
                const uint8_t* g = blk + nib + 32 * (j / 2);
                const int sh = 4 * (j % 2);
                uint8_t* o = dq + (int64_t)(8 * sb + j) * 16;
                for (int i = 0; i < 16; ++i)
                    o[i] = (uint8_t)(((g[i] >> sh) & 15) | (((g[i + 16] >> sh) & 15) << 4));
            }
        }
    } else {  // kQ6_K
        std::memset(dq, 0, (size_t)nb * 24);
        for (int sb = 0; sb < K / 256; ++sb) {
            const uint8_t* blk = src + (int64_t)sb * 210;
            for (int e = 0; e < 256; ++e) {
                const int h = e / 128, t = (e % 128) / 32, l = e % 32;
                const int lo = (blk[64 * h + 32 * (t % 2) + l] >> (4 * (t / 2))) & 15;
                const int hi = (blk[128 + 32 * h + l] >> (2 * t)) & 3;
                const int b = 8 * sb + e / 32, i = e % 32, ii = i & 15;
                dq[(int64_t)b * 16 + ii] |= (uint8_t)(lo << (i < 16 ? 0 : 4));
                dq[(int64_t)nb * 16 + (int64_t)b * 8 + 4 * (i / 16) + (ii & 3)] |= (uint8_t)(hi << (2 * (ii >> 2)));
            }
            std::memcpy(dsc + 16 * sb, blk + 192, 16);                 // scales of blocks 8sb..8sb+7
            std::memcpy(dsc + 2 * nb + 2 * sb, blk + 208, 2);          // d
        }
    }
}

// bytes of one block for the several-sequence layouts (Q8_0 / Q4_0 only)
int block_bytes(int qtype) { return qtype == kQ8_0 ? 34 : 18; }

}  // namespace

// Working memory of one step: the residual stream, q, the attention output,
// the FFN hidden vector, the matrix-core path's activation digits, the
// attention chunks' partial states and counts, and the LM head's per-workgroup
// argmax candidates and counts.  The model's own buffers, or (the
// allocation-free step) slices of the device scratch array.
struct StepBufs {
    float *x = nullptr, *q = nullptr, *o = nullptr, *h = nullptr;
    uint8_t* xfrag = nullptr;
    float* attn_part = nullptr;
    int* attn_cnt = nullptr;
    float* lm_pval = nullptr;
    int* lm_pidx = nullptr;
    int* lm_cnt = nullptr;
};

struct lm_model {
    lm_config cfg{};
    hipStream_t stream = nullptr;
    bool own_stream = false;
    hipStream_t copy_stream = nullptr;
    std::string err;

    int64_t H = 0, F = 0, V = 0, nq = 0, nkv = 0, hd = 0, qrows = 0, kvrows = 0;
    int64_t blob_bytes = 0;
    MatOff mo[M_COUNT]{};
    int64_t lm_q_bytes = 0, lm_sc_bytes = 0, lm_sct_bytes = 0, lm_qf_bytes = 0;
    bool batched = false;                 // max_seqs >= 2: MFMA path for 2..4 sequences
    int max_chunks = 0;
    int gemv_max_blocks = 1024;
    int lm_grid = 0;

    // device memory
    // weight residency: layers 0..n_res-1 live in HBM, layers n_res..L-1 in a
    // pinned host arena, each copied into one of two HBM buffers when used
    int n_res = 0;
    uint8_t* d_layers = nullptr;          // resident blobs [n_res][blob]
    uint8_t* d_sbuf[2] = {nullptr, nullptr};
    uint8_t* h_arena = nullptr;           // pinned blobs [L - n_res][blob] (layer n_res first)
    uint8_t* h_arena_alloc = nullptr;     // the allocation h_arena lies in (it may start later in it)
    uint8_t* h_stage = nullptr;           // pinned staging for uploads
    int64_t stage_bytes = 0;
    float* d_norms = nullptr;             // [L][2][H]
    uint16_t* d_embd = nullptr;
    float* d_out_norm = nullptr;
    uint8_t* d_lm_q = nullptr;
    uint16_t* d_lm_sc = nullptr;
    uint16_t* d_lm_sct = nullptr;
    uint8_t* d_lm_qf = nullptr;           // LM head fragment copy (several-sequence models)
    uint8_t* d_xfrag = nullptr;           // activation operands of the MFMA path
    __half* d_k = nullptr;                // [L][S][nkv][max_ctx][hd]
    __half* d_v = nullptr;
    float *d_x = nullptr, *d_q = nullptr, *d_o = nullptr, *d_h = nullptr, *d_logits = nullptr;
    int *d_tokens = nullptr, *d_argmax = nullptr, *d_pos = nullptr;
    float *d_cos = nullptr, *d_sin = nullptr;
    float* d_attn_part = nullptr;
    int* d_attn_cnt = nullptr;            // [max_seqs][nkv][attn_cnt_lines][kCntStride] attention chunk counters
    float* d_lm_pval = nullptr;
    int* d_lm_pidx = nullptr;
    int* d_lm_cnt = nullptr;
    float* d_sink = nullptr;
    float* d_dbg = nullptr;               // debug dequant rows

    int n_cus = 0;
    int device = 0;                       // the device current at creation
    int64_t dbg_floats = 0;
    StepBufs sb;                          // the buffers the step being enqueued uses

    std::vector<uint8_t> layer_loaded;
    bool global_loaded = false;
    std::vector<int> pos;
    bool streaming = false;               // n_res < L
    // layer skip: skipped layers compute nothing (their input is their output)
    std::vector<uint8_t> skip;
    bool any_skip = false;
    std::vector<int> str_list;            // the streamed layers a step computes, in order
    std::vector<int> str_idx;             // layer -> index in str_list, or -1
    // one step's overrides (self-speculative rounds): positions from opt_pos,
    // every column on sequence 0's cache, positions not advanced, layers from
    // opt_limit on skipped; opt_need = the longest context among the columns
    bool opt_active = false;
    const int* opt_pos = nullptr;
    bool opt_shared_kv = false, opt_advance = true;
    int opt_limit = 0, opt_need = 0;
    int* d_spec = nullptr;                // [8] a round's tokens t0, d1..dk; [8..15] verify argmax
    int* d_vpos = nullptr;                // [4] verify positions
    // layer similarity recording (calibration of the skip list)
    bool sim_on = false;
    double* d_sim = nullptr;              // [L][2]: sum of input/output cosines, records
    float* d_xin = nullptr;               // [max_seqs][H] a layer's input
    bool use_graph = true;

    // streaming pipeline state
    hipEvent_t ev_copied[2] = {nullptr, nullptr};
    hipEvent_t ev_consumed[2] = {nullptr, nullptr};
    bool prefetched[2] = {false, false};   // the next step's first / second streamed layer is copied
    // serial streaming (lm_stream_mode 2): a layer's copy starts when every
    // kernel before it has finished (ev_serial on the compute stream), and
    // nothing is copied ahead: copy, compute, copy, compute
    bool stream_serial = false;
    hipEvent_t ev_serial = nullptr;

    struct Pending { int kind; hipEvent_t a, b; };
    struct GraphEntry {
        int n_seq;
        int chunks;                       // attention grid (attn_grid_chunks at capture)
        const int* tok;
        float* logits;
        int* argmax;
        hipGraphExec_t exec;
        std::vector<Pending> timers;      // event pairs recorded inside the graph (timing mode 2)
        std::vector<hipEvent_t> owned;    // those events, destroyed with the graph
    };
    std::vector<GraphEntry> graphs;

    // kernel timing
    int timing = 0;                       // 0 off, 1 eager steps with events, 2 events inside the graph
    hipError_t timer_err = hipSuccess;    // first failed timing call (reported by the step)
    int only_kind = -1;                   // >= 0 while capturing a one-family timing graph
    // timing mode 2: the graph nodes each timed scope captured (its last node and
    // the node before it); event-record nodes are inserted around them afterwards
    struct CapScope { int kind; hipGraphNode_t before, last; };
    std::vector<CapScope> cap_scopes;
    int64_t kcount[LM_K_COUNT] = {};
    double kms[LM_K_COUNT] = {};
    std::vector<Pending> pending;
    std::vector<hipEvent_t> ev_pool;
    size_t ev_used = 0;

    std::vector<void*> dev_allocs;
    std::vector<void*> host_allocs;
};

// ---------------------------------------------------------------------------
// error helpers
// ---------------------------------------------------------------------------
static lm_status fail(lm_model* m, lm_status st, const char* fmt, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (m) m->err = buf;
    else g_create_error = buf;
    return st;
}

#define HIPTRY(m, call)                                                                    \
    do {                                                                                   \
        hipError_t _e = (call);                                                            \
        if (_e != hipSuccess)                                                              \
            return fail((m), LM_E_HIP, "%s failed: %s (%d)", #call, hipGetErrorString(_e), \
                        (int)_e);                                                          \
    } while (0)

// Allocation fault injection (lm_debug_fail_alloc): the allocation whose
// process-wide number equals g_fail_at fails as if the memory were exhausted.
static bool fault_alloc_now() {
    const long n = ++g_alloc_count;
    long at = g_fail_at.load();
    return at > 0 && n == at && g_fail_at.compare_exchange_strong(at, 0L);
}

static lm_status dev_alloc(lm_model* m, void** p, int64_t bytes, const char* what) {
    *p = nullptr;
    if (bytes <= 0) bytes = kAlign;
    if (fault_alloc_now())
        return fail(m, LM_E_OOM, "device allocation of %s (%lld bytes) failed: injected by LM_FAULT_ALLOC_AT",
                    what, (long long)bytes);
    hipError_t e = hipMalloc(p, (size_t)bytes);
    if (e != hipSuccess) {
        *p = nullptr;
        (void)hipGetLastError();
        return fail(m, LM_E_OOM, "hipMalloc of %s (%lld bytes) failed: %s", what, (long long)bytes,
                    hipGetErrorString(e));
    }
    m->dev_allocs.push_back(*p);
    return LM_OK;
}

static lm_status host_alloc(lm_model* m, void** p, int64_t bytes, const char* what) {
    *p = nullptr;
    if (fault_alloc_now())
        return fail(m, LM_E_OOM, "pinned host allocation of %s (%lld bytes) failed: injected by LM_FAULT_ALLOC_AT",
                    what, (long long)bytes);
    hipError_t e = hipHostMalloc(p, (size_t)bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
        *p = nullptr;
        (void)hipGetLastError();
        return fail(m, LM_E_OOM, "hipHostMalloc of %s (%lld bytes) failed: %s", what, (long long)bytes,
                    hipGetErrorString(e));
    }
    m->host_allocs.push_back(*p);
    return LM_OK;
}

static void dev_free(lm_model* m, void* p) {
    if (!p) return;
    (void)hipFree(p);
    m->dev_allocs.erase(std::remove(m->dev_allocs.begin(), m->dev_allocs.end(), p), m->dev_allocs.end());
}

static void host_free(lm_model* m, void* p) {
    if (!p) return;
    (void)hipHostFree(p);
    m->host_allocs.erase(std::remove(m->host_allocs.begin(), m->host_allocs.end(), p), m->host_allocs.end());
}

static void release_all(lm_model* m) {
    if (m->stream) (void)hipStreamSynchronize(m->stream);
    if (m->copy_stream) (void)hipStreamSynchronize(m->copy_stream);
    for (auto& g : m->graphs) (void)hipGraphExecDestroy(g.exec);
    m->graphs.clear();
    for (auto e : m->ev_pool) (void)hipEventDestroy(e);
    m->ev_pool.clear();
    for (int i = 0; i < 2; ++i) {
        if (m->ev_copied[i]) (void)hipEventDestroy(m->ev_copied[i]);
        if (m->ev_consumed[i]) (void)hipEventDestroy(m->ev_consumed[i]);
        m->ev_copied[i] = m->ev_consumed[i] = nullptr;
    }
    if (m->ev_serial) (void)hipEventDestroy(m->ev_serial);
    m->ev_serial = nullptr;
    for (void* p : m->dev_allocs) (void)hipFree(p);
    m->dev_allocs.clear();
    for (void* p : m->host_allocs) (void)hipHostFree(p);
    m->host_allocs.clear();
    if (m->copy_stream) (void)hipStreamDestroy(m->copy_stream);
    m->copy_stream = nullptr;
    if (m->own_stream && m->stream) (void)hipStreamDestroy(m->stream);
    m->stream = nullptr;
}

static void rebuild_stream_order(lm_model* m);

// ---------------------------------------------------------------------------
// configuration checks (no HIP call before these pass)
// ---------------------------------------------------------------------------
static lm_status check_config(const lm_config* c) {
    auto bad = [](const char* what, long long got, const char* expect) {
        return fail(nullptr, LM_E_ARG, "bad config: %s = %lld; expected %s", what, got, expect);
    };
    if (!c) return fail(nullptr, LM_E_ARG, "bad config: NULL pointer");
    if (c->qtype != LM_Q8_0 && c->qtype != LM_Q4_0 && c->qtype != LM_Q4_K && c->qtype != LM_Q5_K &&
        c->qtype != LM_Q6_K)
        return bad("qtype", c->qtype, "2 (Q4_0), 8 (Q8_0), 12 (Q4_K), 13 (Q5_K) or 14 (Q6_K)");
    if (is_kquant(c->qtype)) {
        // 256-weight super-blocks along every GEMV input; one sequence per step
        if (c->hidden % 256) return bad("hidden", c->hidden, "a multiple of 256 for the K formats");
        if (c->ffn % 256) return bad("ffn", c->ffn, "a multiple of 256 for the K formats");
        if ((int64_t)c->n_heads * c->head_dim % 256)
            return bad("n_heads * head_dim", (long long)c->n_heads * c->head_dim, "a multiple of 256 for the K formats");
        if (c->max_seqs != 1) return bad("max_seqs", c->max_seqs, "1 for the K formats (one sequence per step)");
    }
    if (c->vocab < 2 || c->vocab % 2) return bad("vocab", c->vocab, "an even number >= 2");
    if (c->hidden < 32 || c->hidden % 32) return bad("hidden", c->hidden, "a positive multiple of 32");
    if (c->n_layers < 1) return bad("n_layers", c->n_layers, ">= 1");
    if (c->n_heads < 1) return bad("n_heads", c->n_heads, ">= 1");
    if (c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads)
        return bad("n_kv_heads", c->n_kv_heads, "a divisor of n_heads");
    if (c->n_heads / c->n_kv_heads > 8) return bad("n_heads / n_kv_heads", c->n_heads / c->n_kv_heads, "<= 8");
    if (c->head_dim != 64 && c->head_dim != 128) return bad("head_dim", c->head_dim, "64 or 128");
    if (c->ffn < 32 || c->ffn % 32) return bad("ffn", c->ffn, "a positive multiple of 32");
    if (c->max_ctx < 1) return bad("max_ctx", c->max_ctx, ">= 1");
    if (c->max_seqs < 1 || c->max_seqs > 4) return bad("max_seqs", c->max_seqs, "1..4");
    // 2..4 sequences: an RMSNorm-gained input (QKV, gate/up, LM head: K =
    // hidden) has its digits staged by each GEMV workgroup in LDS, at most
    // 6144 columns (lm_kernels.hip, kMbLdsMaxK)
    if (c->max_seqs >= 2 && c->hidden > 6144)
        return bad("hidden", c->hidden, "<= 6144 when max_seqs >= 2");
    if (!(c->rms_eps >= 0.0) || !std::isfinite(c->rms_eps))
        return fail(nullptr, LM_E_ARG, "bad config: rms_eps = %g; expected a finite value >= 0", c->rms_eps);
    if (!(c->rope_theta > 0.0) || !std::isfinite(c->rope_theta))
        return fail(nullptr, LM_E_ARG, "bad config: rope_theta = %g; expected a finite value > 0", c->rope_theta);
    const int64_t kmax = std::max<int64_t>({c->hidden, c->ffn, (int64_t)c->n_heads * c->head_dim});
    const int64_t lds = kmax * 4 + kmax / 32 * 4;
    if (lds > 150 * 1024)
        return fail(nullptr, LM_E_ARG, "bad config: widest GEMV input has %lld columns (%lld bytes of LDS); "
                    "expected at most %d bytes", (long long)kmax, (long long)lds, 150 * 1024);
    return LM_OK;
}

static void layout(lm_model* m) {
    const lm_config& c = m->cfg;
    m->H = c.hidden; m->F = c.ffn; m->V = c.vocab;
    m->nq = c.n_heads; m->nkv = c.n_kv_heads; m->hd = c.head_dim;
    m->qrows = m->nq * m->hd;
    m->kvrows = m->nkv * m->hd;
    const int qt = c.qtype;
    int64_t off = 0;
    const int64_t NK[M_COUNT][2] = {{m->qrows + 2 * m->kvrows, m->H},
                                    {m->H, m->qrows},
                                    {2 * m->F, m->H},
                                    {m->H, m->F}};
    for (int i = 0; i < M_COUNT; ++i) {
        m->mo[i].N = (int)NK[i][0];
        m->mo[i].K = (int)NK[i][1];
        m->mo[i].q = off;
        off = align_up(off + qmat_qbytes(qt, NK[i][0], NK[i][1]));
        m->mo[i].sc = off;
        off = align_up(off + qmat_sbytes(qt, NK[i][0], NK[i][1]));
        m->mo[i].sct = -1;
        m->mo[i].qf = -1;
        if (m->batched) {
            m->mo[i].sct = off;
            off = align_up(off + sct_bytes(NK[i][0], NK[i][1]));
            m->mo[i].qf = off;
            off = align_up(off + qfrag_bytes(qt, NK[i][0], NK[i][1]));
        }
    }
    m->blob_bytes = off;
    m->lm_q_bytes = align_up(qmat_qbytes(qt, m->V, m->H));
    m->lm_sc_bytes = align_up(qmat_sbytes(qt, m->V, m->H));
    m->lm_sct_bytes = m->batched ? align_up(sct_bytes(m->V, m->H)) : 0;
    m->lm_qf_bytes = m->batched ? align_up(qfrag_bytes(qt, m->V, m->H)) : 0;
    m->max_chunks = (c.max_ctx + kAttnChunk - 1) / kAttnChunk;
}

static QMat mat_at(const lm_model* m, const uint8_t* blob, int which) {
    QMat w;
    w.q = blob + m->mo[which].q;
    w.sc = (const uint16_t*)(blob + m->mo[which].sc);
    w.sct = m->mo[which].sct >= 0 ? (const uint16_t*)(blob + m->mo[which].sct) : nullptr;
    w.qf = m->mo[which].qf >= 0 ? blob + m->mo[which].qf : nullptr;
    w.N = m->mo[which].N;
    w.K = m->mo[which].K;
    return w;
}

static QMat lm_head_mat(const lm_model* m) {
    QMat w;
    w.q = m->d_lm_q;
    w.sc = m->d_lm_sc;
    w.sct = m->d_lm_sct;
    w.qf = m->d_lm_qf;
    w.N = (int)m->V;
    w.K = (int)m->H;
    return w;
}

static int64_t kv_layer_elems(const lm_model* m) {
    return (int64_t)m->cfg.max_seqs * m->nkv * m->cfg.max_ctx * m->hd;
}

static int64_t kv_seq_elems(const lm_model* m) { return m->nkv * (int64_t)m->cfg.max_ctx * m->hd; }

// ---------------------------------------------------------------------------
// create / destroy
// ---------------------------------------------------------------------------
extern "C" lm_status lm_model_create(const lm_config* cfg, void* hip_stream, lm_model** out) {
    g_create_error.clear();
    if (!out) return fail(nullptr, LM_E_ARG, "lm_model_create: out is NULL");
    *out = nullptr;
    lm_status st = check_config(cfg);
    if (st != LM_OK) return st;

    lm_model* m = new (std::nothrow) lm_model();
    if (!m) return fail(nullptr, LM_E_OOM, "lm_model_create: host allocation failed");
    m->cfg = *cfg;
    m->batched = cfg->max_seqs >= 2;
    layout(m);
    m->layer_loaded.assign(cfg->n_layers, 0);
    m->pos.assign(cfg->max_seqs, 0);

    auto bail = [&](lm_status s) {
        g_create_error = m->err;
        release_all(m);
        delete m;
        return s;
    };
#define CREATE_TRY(expr)                      \
    do {                                      \
        lm_status _s = (expr);                \
        if (_s != LM_OK) return bail(_s);     \
    } while (0)
#define CREATE_HIP(call)                                                                   \
    do {                                                                                   \
        hipError_t _e = (call);                                                            \
        if (_e != hipSuccess) {                                                            \
            fail(m, LM_E_HIP, "%s failed: %s (%d)", #call, hipGetErrorString(_e), (int)_e); \
            return bail(LM_E_HIP);                                                         \
        }                                                                                  \
    } while (0)

    int ndev = 0;
    CREATE_HIP(hipGetDeviceCount(&ndev));
    if (hip_stream) {
        m->stream = (hipStream_t)hip_stream;
        m->own_stream = false;
    } else {
        CREATE_HIP(hipStreamCreateWithFlags(&m->stream, hipStreamNonBlocking));
        m->own_stream = true;
    }
    CREATE_HIP(hipStreamCreateWithFlags(&m->copy_stream, hipStreamNonBlocking));
    for (int i = 0; i < 2; ++i) {
        CREATE_HIP(hipEventCreateWithFlags(&m->ev_copied[i], hipEventDisableTiming));
        CREATE_HIP(hipEventCreateWithFlags(&m->ev_consumed[i], hipEventDisableTiming));
    }
    CREATE_HIP(hipEventCreateWithFlags(&m->ev_serial, hipEventDisableTiming));
    {
        int dev = 0, ncu = 0;
        CREATE_HIP(hipGetDevice(&dev));
        CREATE_HIP(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
        m->gemv_max_blocks = std::max(64, ncu * 4);
        m->n_cus = ncu;
        m->device = dev;
    }

    const lm_config& c = *cfg;
    const int S = c.max_seqs;
    const int64_t L = c.n_layers;
    CREATE_TRY(dev_alloc(m, (void**)&m->d_layers, L * m->blob_bytes, "layer weights"));
    m->n_res = (int)L;
    m->skip.assign((size_t)L, 0);
    rebuild_stream_order(m);
    CREATE_TRY(dev_alloc(m, (void**)&m->d_norms, L * 2 * m->H * 4, "norm gains"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_embd, m->V * m->H * 2, "token embedding"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_out_norm, m->H * 4, "output norm"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_lm_q, m->lm_q_bytes, "LM head quants"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_lm_sc, m->lm_sc_bytes, "LM head scales"));
    if (m->batched) {
        CREATE_TRY(dev_alloc(m, (void**)&m->d_lm_sct, m->lm_sct_bytes, "LM head transposed scales"));
        CREATE_TRY(dev_alloc(m, (void**)&m->d_lm_qf, m->lm_qf_bytes, "LM head matrix-core fragments"));
        const int64_t kmax = std::max<int64_t>({m->H, m->qrows, m->F});
        CREATE_TRY(dev_alloc(m, (void**)&m->d_xfrag, xfrag_bytes(kmax), "activation fragments"));
        CREATE_HIP(hipMemsetAsync(m->d_xfrag, 0, (size_t)xfrag_bytes(kmax), m->stream));
    }
    CREATE_TRY(dev_alloc(m, (void**)&m->d_k, L * kv_layer_elems(m) * 2, "K cache"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_v, L * kv_layer_elems(m) * 2, "V cache"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_x, S * m->H * 4, "residual"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_q, S * m->qrows * 4, "q"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_o, S * m->qrows * 4, "attention output"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_h, S * m->F * 4, "ffn hidden"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_logits, S * m->V * 4, "logits"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_tokens, S * 4, "tokens"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_argmax, S * 4, "argmax"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_pos, S * 4, "positions"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_cos, (int64_t)c.max_ctx * (m->hd / 2) * 4, "rope cos"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_sin, (int64_t)c.max_ctx * (m->hd / 2) * 4, "rope sin"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_attn_part,
                         (int64_t)S * m->nq * m->max_chunks * (m->hd + 2) * 4, "attention partials"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_lm_pval, (int64_t)S * m->gemv_max_blocks * 4, "argmax partials"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_lm_pidx, (int64_t)S * m->gemv_max_blocks * 4, "argmax partial ids"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_lm_cnt, (int64_t)S * 4, "argmax counters"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_attn_cnt, (int64_t)S * m->nkv * attn_cnt_lines(m->max_chunks) * kCntStride * 4,
                         "attention chunk counters"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_sink, 4096 * 4, "sink"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_sim, (int64_t)L * 2 * 8, "layer similarity sums"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_spec, 16 * 4, "speculative round tokens"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_vpos, 4 * 4, "verify positions"));
    CREATE_TRY(dev_alloc(m, (void**)&m->d_xin, (int64_t)S * m->H * 4, "layer input copy"));
    m->dbg_floats = std::max<int64_t>({m->H, m->F, m->qrows}) * 64;
    CREATE_TRY(dev_alloc(m, (void**)&m->d_dbg, m->dbg_floats * 4, "debug rows"));
    m->stage_bytes = std::min<int64_t>(64ll << 20, std::max<int64_t>(m->blob_bytes, m->lm_q_bytes + m->lm_sc_bytes));
    m->stage_bytes = std::max<int64_t>(m->stage_bytes, 4 * (m->H * 34 / 32 + 64));
    CREATE_TRY(host_alloc(m, (void**)&m->h_stage, m->stage_bytes, "upload staging"));

    m->sb.x = m->d_x;
    m->sb.q = m->d_q;
    m->sb.o = m->d_o;
    m->sb.h = m->d_h;
    m->sb.xfrag = m->d_xfrag;
    m->sb.attn_part = m->d_attn_part;
    m->sb.attn_cnt = m->d_attn_cnt;
    m->sb.lm_pval = m->d_lm_pval;
    m->sb.lm_pidx = m->d_lm_pidx;
    m->sb.lm_cnt = m->d_lm_cnt;

    // zero what must start at zero (counters, caches, positions)
    CREATE_HIP(hipMemsetAsync(m->d_lm_cnt, 0, (size_t)S * 4, m->stream));
    CREATE_HIP(hipMemsetAsync(m->d_attn_cnt, 0, (size_t)S * m->nkv * attn_cnt_lines(m->max_chunks) * kCntStride * 4,
                              m->stream));
    CREATE_HIP(hipMemsetAsync(m->d_pos, 0, (size_t)S * 4, m->stream));
    CREATE_HIP(hipMemsetAsync(m->d_k, 0, (size_t)(L * kv_layer_elems(m) * 2), m->stream));
    CREATE_HIP(hipMemsetAsync(m->d_v, 0, (size_t)(L * kv_layer_elems(m) * 2), m->stream));

    // RoPE table: angle p * theta^(-2i/hd) evaluated in fp64, stored fp32
    {
        const int half = (int)(m->hd / 2);
        std::vector<float> cs((size_t)c.max_ctx * half), sn((size_t)c.max_ctx * half);
        for (int p = 0; p < c.max_ctx; ++p)
            for (int i = 0; i < half; ++i) {
                const double f = std::pow(c.rope_theta, -2.0 * i / (double)m->hd);
                const double a = (double)p * f;
                cs[(size_t)p * half + i] = (float)std::cos(a);
                sn[(size_t)p * half + i] = (float)std::sin(a);
            }
        CREATE_HIP(hipMemcpy(m->d_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice));
        CREATE_HIP(hipMemcpy(m->d_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice));
    }
    CREATE_HIP(hipStreamSynchronize(m->stream));
#undef CREATE_TRY
#undef CREATE_HIP
    *out = m;
    return LM_OK;
}

extern "C" void lm_model_destroy(lm_model* m) {
    if (!m) return;
    release_all(m);
    delete m;
}

extern "C" const char* lm_last_error(const lm_model* m) {
    return m ? m->err.c_str() : g_create_error.c_str();
}

extern "C" void* lm_stream(const lm_model* m) { return m ? (void*)m->stream : nullptr; }

// ---------------------------------------------------------------------------
// weight upload
// ---------------------------------------------------------------------------
// Repacks rows [0, N) of one matrix, whose row r comes from src_row(r), into
// the device layout at (dq, dsc).  dst_host: the destination is host memory
// (the pinned arena) and is written directly; otherwise rows go through the
// pinned staging buffer in chunks.
template <class RowFn>
static lm_status upload_matrix(lm_model* m, int N, int K, RowFn src_row, uint8_t* dq, uint16_t* dsc,
                               bool dst_host) {
    const int qt = m->cfg.qtype;
    const int64_t rq = qmat_qbytes(qt, 1, K), rs = qmat_srow(qt, K);
    // Q8_0 / Q4_0: scales of a row pair interleaved (N is even); the K formats: a row's scales contiguous
    const bool pairs = (qt == kQ8_0 || qt == kQ4_0) && kScPairs;
    auto srow_at = [&](uint8_t* base, int64_t r) { return pairs ? base + (r >> 1) * 2 * rs + (r & 1) * 2 : base + r * rs; };
    uint8_t* dsb = (uint8_t*)dsc;
    if (dst_host) {
        parallel_rows(N, [&](int64_t a, int64_t b) {
            for (int64_t r = a; r < b; ++r) repack_row(qt, src_row(r), K, dq + r * rq, srow_at(dsb, r));
        });
        return LM_OK;
    }
    const int64_t rows_per = std::max<int64_t>(2, m->stage_bytes / (rq + rs)) & ~(int64_t)1;   // whole row pairs
    for (int64_t r0 = 0; r0 < N; r0 += rows_per) {
        const int64_t n = std::min<int64_t>(rows_per, N - r0);
        uint8_t* sq = m->h_stage;
        uint8_t* ss = m->h_stage + n * rq;
        parallel_rows(n, [&](int64_t a, int64_t b) {
            for (int64_t r = a; r < b; ++r) repack_row(qt, src_row(r0 + r), K, sq + r * rq, srow_at(ss, r));
        });
        HIPTRY(m, hipMemcpyAsync(dq + r0 * rq, sq, (size_t)(n * rq), hipMemcpyHostToDevice, m->stream));
        HIPTRY(m, hipMemcpyAsync(dsb + r0 * rs, ss, (size_t)(n * rs), hipMemcpyHostToDevice, m->stream));
        HIPTRY(m, hipStreamSynchronize(m->stream));
    }
    return LM_OK;
}

// The grouped copy of a matrix's block scales used by the MFMA path:
// dst[t][b/4][i][b%4] = scale of row 16t+i, block b (zero past the last row and block).
template <class RowFn>
static lm_status upload_sct(lm_model* m, int N, int K, RowFn src_row, uint16_t* dst, bool dst_host) {
    const int64_t nb = K / 32, tiles = (N + 15) / 16, bb = block_bytes(m->cfg.qtype), ng = (nb + 3) / 4;
    const int64_t n = sct_bytes(N, K) / 2;
    std::vector<uint16_t> tmp;
    uint16_t* t = dst;
    if (!dst_host) {
        tmp.assign((size_t)n, 0);
        t = tmp.data();
    } else {
        std::memset(t, 0, (size_t)n * 2);
    }
    parallel_rows(tiles, [&](int64_t a, int64_t b) {
        for (int64_t tile = a; tile < b; ++tile)
            for (int i = 0; i < 16; ++i) {
                const int64_t r = tile * 16 + i;
                if (r >= N) continue;
                const uint8_t* src = src_row(r);
                for (int64_t k = 0; k < nb; ++k)
                    t[((tile * ng + k / 4) * 16 + i) * 4 + k % 4] = (uint16_t)(src[k * bb] | (src[k * bb + 1] << 8));
            }
    });
    if (!dst_host) HIPTRY(m, hipMemcpy(dst, t, (size_t)n * 2, hipMemcpyHostToDevice));
    return LM_OK;
}

// The matrix-core fragment copy of a matrix's quants (layout: lm_internal.h,
// qfrag_bytes): per 16-row tile and group of blocks, lane l = 16g + j holds
// row j, columns 8g..8g+7 of each block of the group.  Zero past the last row
// and past the last block.
template <class RowFn>
static lm_status upload_frag(lm_model* m, int N, int K, RowFn src_row, uint8_t* dst, bool dst_host) {
    const int qt = m->cfg.qtype;
    const int64_t nb = K / 32, tiles = (N + 15) / 16, bb = block_bytes(qt);
    const int per = qfrag_blocks(qt);                    // blocks per 16-byte lane slice
    const int64_t ngrp = (nb + per - 1) / per;
    const int64_t bytes = qfrag_bytes(qt, N, K);
    std::vector<uint8_t> tmp;
    uint8_t* t = dst;
    if (!dst_host) {
        tmp.assign((size_t)bytes, 0);
        t = tmp.data();
    } else {
        std::memset(t, 0, (size_t)bytes);
    }
    parallel_rows(tiles, [&](int64_t a, int64_t b) {
        for (int64_t tile = a; tile < b; ++tile)
            for (int j = 0; j < 16; ++j) {
                const int64_t r = tile * 16 + j;
                if (r >= N) continue;
                const uint8_t* src = src_row(r);
                for (int64_t blk = 0; blk < nb; ++blk) {
                    const uint8_t* qs = src + blk * bb + 2;      // past the fp16 scale
                    const int64_t grp = blk / per, k = blk % per;
                    for (int g = 0; g < 4; ++g) {
                        uint8_t* lane = t + ((tile * ngrp + grp) * 64 + 16 * g + j) * 16;
                        if (qt == kQ8_0) {
                            std::memcpy(lane + 8 * k, qs + 8 * g, 8);
                        } else {
                            // byte i: nibble of column 8g+i (low), of column 8g+4+i (high)
                            auto nib = [&](int c) { return c < 16 ? (qs[c] & 15) : (qs[c - 16] >> 4); };
                            for (int i = 0; i < 4; ++i)
                                lane[4 * k + i] = (uint8_t)(nib(8 * g + i) | (nib(8 * g + 4 + i) << 4));
                        }
                    }
                }
            }
    });
    if (!dst_host) HIPTRY(m, hipMemcpy(dst, t, (size_t)bytes, hipMemcpyHostToDevice));
    return LM_OK;
}

// residency: layers n_res..L-1 are streamed through the two HBM buffers,
// alternating between them in order
static bool layer_streamed(const lm_model* m, int l) { return l >= m->n_res; }
// the streamed layers a step computes take the two buffers in turn
static int stream_slot(const lm_model* m, int l) { return m->str_idx[l] & 1; }
static void rebuild_stream_order(lm_model* m) {
    const int L = m->cfg.n_layers;
    m->str_list.clear();
    m->str_idx.assign((size_t)L, -1);
    for (int l = m->n_res; l < L; ++l)
        if (!m->skip[l]) {
            m->str_idx[l] = (int)m->str_list.size();
            m->str_list.push_back(l);
        }
}
static uint8_t* host_blob(lm_model* m, int l) { return m->h_arena + (int64_t)(l - m->n_res) * m->blob_bytes; }

static void invalidate_graphs(lm_model* m) {
    for (auto& g : m->graphs) {
        (void)hipGraphExecDestroy(g.exec);
        for (hipEvent_t e : g.owned) (void)hipEventDestroy(e);
    }
    m->graphs.clear();
}

extern "C" lm_status lm_load_layer_weights(lm_model* m, int32_t layer, const lm_layer_weights* w) {
    if (!m) return LM_E_ARG;
    if (layer < 0 || layer >= m->cfg.n_layers)
        return fail(m, LM_E_ARG, "lm_load_layer_weights: layer = %d; expected 0..%d", layer, m->cfg.n_layers - 1);
    if (!w || !w->attn_norm || !w->ffn_norm || !w->wq || !w->wk || !w->wv || !w->wo || !w->w_gate ||
        !w->w_up || !w->w_down)
        return fail(m, LM_E_ARG, "lm_load_layer_weights: a weight pointer is NULL (layer %d)", layer);
    HIPTRY(m, hipStreamSynchronize(m->stream));
    HIPTRY(m, hipStreamSynchronize(m->copy_stream));
    const int qt = m->cfg.qtype;
    const int64_t H = m->H, F = m->F;
    const int64_t rowH = gguf_row_bytes(qt, H), rowQ = gguf_row_bytes(qt, m->qrows), rowF = gguf_row_bytes(qt, F);
    const uint8_t *wq = (const uint8_t*)w->wq, *wk = (const uint8_t*)w->wk, *wv = (const uint8_t*)w->wv;
    const uint8_t *wo = (const uint8_t*)w->wo, *wg = (const uint8_t*)w->w_gate, *wu = (const uint8_t*)w->w_up;
    const uint8_t* wd = (const uint8_t*)w->w_down;
    const int64_t qr = m->qrows, kr = m->kvrows;
    const bool host = layer_streamed(m, layer);
    uint8_t* blob = host ? host_blob(m, layer) : m->d_layers + (int64_t)layer * m->blob_bytes;
    auto dq = [&](int i) { return blob + m->mo[i].q; };
    auto ds = [&](int i) { return (uint16_t*)(blob + m->mo[i].sc); };
    auto src_qkv = [&](int64_t r) {
        if (r < qr) return wq + r * rowH;
        if (r < qr + kr) return wk + (r - qr) * rowH;
        return wv + (r - qr - kr) * rowH;
    };
    auto src_wo = [&](int64_t r) { return wo + r * rowQ; };
    // gate and up rows interleaved: device row 2i = gate i, 2i+1 = up i
    auto src_gu = [&](int64_t r) { return (r & 1) ? wu + (r >> 1) * rowH : wg + (r >> 1) * rowH; };
    auto src_down = [&](int64_t r) { return wd + r * rowF; };
    lm_status st;
    st = upload_matrix(m, m->mo[M_QKV].N, (int)H, src_qkv, dq(M_QKV), ds(M_QKV), host);
    if (st != LM_OK) return st;
    st = upload_matrix(m, (int)H, (int)m->qrows, src_wo, dq(M_WO), ds(M_WO), host);
    if (st != LM_OK) return st;
    st = upload_matrix(m, (int)(2 * F), (int)H, src_gu, dq(M_GU), ds(M_GU), host);
    if (st != LM_OK) return st;
    st = upload_matrix(m, (int)H, (int)F, src_down, dq(M_DOWN), ds(M_DOWN), host);
    if (st != LM_OK) return st;
    if (m->batched) {
        auto dt = [&](int i) { return (uint16_t*)(blob + m->mo[i].sct); };
        if ((st = upload_sct(m, m->mo[M_QKV].N, (int)H, src_qkv, dt(M_QKV), host)) != LM_OK) return st;
        if ((st = upload_sct(m, (int)H, (int)m->qrows, src_wo, dt(M_WO), host)) != LM_OK) return st;
        if ((st = upload_sct(m, (int)(2 * F), (int)H, src_gu, dt(M_GU), host)) != LM_OK) return st;
        if ((st = upload_sct(m, (int)H, (int)F, src_down, dt(M_DOWN), host)) != LM_OK) return st;
        auto df = [&](int i) { return blob + m->mo[i].qf; };
        if ((st = upload_frag(m, m->mo[M_QKV].N, (int)H, src_qkv, df(M_QKV), host)) != LM_OK) return st;
        if ((st = upload_frag(m, (int)H, (int)m->qrows, src_wo, df(M_WO), host)) != LM_OK) return st;
        if ((st = upload_frag(m, (int)(2 * F), (int)H, src_gu, df(M_GU), host)) != LM_OK) return st;
        if ((st = upload_frag(m, (int)H, (int)F, src_down, df(M_DOWN), host)) != LM_OK) return st;
    }
    HIPTRY(m, hipMemcpy(m->d_norms + (int64_t)layer * 2 * H, w->attn_norm, H * 4, hipMemcpyHostToDevice));
    HIPTRY(m, hipMemcpy(m->d_norms + ((int64_t)layer * 2 + 1) * H, w->ffn_norm, H * 4, hipMemcpyHostToDevice));
    m->layer_loaded[layer] = 1;
    m->prefetched[0] = m->prefetched[1] = false;
    return LM_OK;
}

extern "C" lm_status lm_load_global_weights(lm_model* m, const uint16_t* tok_embd_f16, const float* out_norm,
                                            const void* lm_head_blocks) {
    if (!m) return LM_E_ARG;
    if (!tok_embd_f16 || !out_norm || !lm_head_blocks)
        return fail(m, LM_E_ARG, "lm_load_global_weights: a pointer is NULL");
    HIPTRY(m, hipStreamSynchronize(m->stream));
    HIPTRY(m, hipMemcpy(m->d_embd, tok_embd_f16, (size_t)(m->V * m->H * 2), hipMemcpyHostToDevice));
    HIPTRY(m, hipMemcpy(m->d_out_norm, out_norm, (size_t)(m->H * 4), hipMemcpyHostToDevice));
    const int64_t rowH = gguf_row_bytes(m->cfg.qtype, m->H);
    const uint8_t* src = (const uint8_t*)lm_head_blocks;
    auto src_row = [&](int64_t r) { return src + r * rowH; };
    lm_status st = upload_matrix(m, (int)m->V, (int)m->H, src_row, m->d_lm_q, m->d_lm_sc, false);
    if (st != LM_OK) return st;
    if (m->batched && (st = upload_sct(m, (int)m->V, (int)m->H, src_row, m->d_lm_sct, false)) != LM_OK) return st;
    if (m->batched && (st = upload_frag(m, (int)m->V, (int)m->H, src_row, m->d_lm_qf, false)) != LM_OK) return st;
    m->global_loaded = true;
    return LM_OK;
}

// ---------------------------------------------------------------------------
// KV cache and positions
// ---------------------------------------------------------------------------
static lm_status check_seq_layer(lm_model* m, const char* fn, int seq, int layer) {
    if (seq < 0 || seq >= m->cfg.max_seqs)
        return fail(m, LM_E_ARG, "%s: seq = %d; expected 0..%d", fn, seq, m->cfg.max_seqs - 1);
    if (layer < 0 || layer >= m->cfg.n_layers)
        return fail(m, LM_E_ARG, "%s: layer = %d; expected 0..%d", fn, layer, m->cfg.n_layers - 1);
    return LM_OK;
}

extern "C" lm_status lm_load_kv(lm_model* m, int32_t seq, int32_t layer, const uint16_t* k, const uint16_t* v,
                                int32_t n_pos) {
    if (!m) return LM_E_ARG;
    lm_status st = check_seq_layer(m, "lm_load_kv", seq, layer);
    if (st != LM_OK) return st;
    if (n_pos < 0 || n_pos > m->cfg.max_ctx)
        return fail(m, LM_E_ARG, "lm_load_kv: n_pos = %d; expected 0..%d (max_ctx)", n_pos, m->cfg.max_ctx);
    if (n_pos > 0 && (!k || !v)) return fail(m, LM_E_ARG, "lm_load_kv: k or v is NULL");
    HIPTRY(m, hipStreamSynchronize(m->stream));
    const int64_t base = (int64_t)layer * kv_layer_elems(m) + (int64_t)seq * kv_seq_elems(m);
    const size_t row = (size_t)n_pos * m->hd * 2;
    for (int g = 0; g < m->nkv && n_pos > 0; ++g) {
        const int64_t off = base + (int64_t)g * m->cfg.max_ctx * m->hd;
        HIPTRY(m, hipMemcpy(m->d_k + off, k + (int64_t)g * n_pos * m->hd, row, hipMemcpyHostToDevice));
        HIPTRY(m, hipMemcpy(m->d_v + off, v + (int64_t)g * n_pos * m->hd, row, hipMemcpyHostToDevice));
    }
    int p = n_pos;
    HIPTRY(m, hipMemcpy(m->d_pos + seq, &p, 4, hipMemcpyHostToDevice));
    m->pos[seq] = n_pos;
    return LM_OK;
}

extern "C" lm_status lm_get_kv(lm_model* m, int32_t seq, int32_t layer, uint16_t* k, uint16_t* v, int32_t n_pos) {
    if (!m) return LM_E_ARG;
    lm_status st = check_seq_layer(m, "lm_get_kv", seq, layer);
    if (st != LM_OK) return st;
    if (n_pos < 0 || n_pos > m->cfg.max_ctx)
        return fail(m, LM_E_ARG, "lm_get_kv: n_pos = %d; expected 0..%d (max_ctx)", n_pos, m->cfg.max_ctx);
    if (n_pos > 0 && (!k || !v)) return fail(m, LM_E_ARG, "lm_get_kv: k or v is NULL");
    HIPTRY(m, hipStreamSynchronize(m->stream));
    const int64_t base = (int64_t)layer * kv_layer_elems(m) + (int64_t)seq * kv_seq_elems(m);
    const size_t row = (size_t)n_pos * m->hd * 2;
    for (int g = 0; g < m->nkv && n_pos > 0; ++g) {
        const int64_t off = base + (int64_t)g * m->cfg.max_ctx * m->hd;
        HIPTRY(m, hipMemcpy(k + (int64_t)g * n_pos * m->hd, m->d_k + off, row, hipMemcpyDeviceToHost));
        HIPTRY(m, hipMemcpy(v + (int64_t)g * n_pos * m->hd, m->d_v + off, row, hipMemcpyDeviceToHost));
    }
    return LM_OK;
}

extern "C" lm_status lm_set_position(lm_model* m, int32_t seq, int32_t pos) {
    if (!m) return LM_E_ARG;
    if (seq < 0 || seq >= m->cfg.max_seqs)
        return fail(m, LM_E_ARG, "lm_set_position: seq = %d; expected 0..%d", seq, m->cfg.max_seqs - 1);
    if (pos < 0 || pos > m->cfg.max_ctx)
        return fail(m, LM_E_ARG, "lm_set_position: pos = %d; expected 0..%d (max_ctx)", pos, m->cfg.max_ctx);
    HIPTRY(m, hipStreamSynchronize(m->stream));
    int p = pos;
    HIPTRY(m, hipMemcpy(m->d_pos + seq, &p, 4, hipMemcpyHostToDevice));
    m->pos[seq] = pos;
    return LM_OK;
}

extern "C" lm_status lm_get_position(const lm_model* m, int32_t seq, int32_t* pos) {
    if (!m || !pos || seq < 0 || seq >= m->cfg.max_seqs) return LM_E_ARG;
    *pos = m->pos[seq];
    return LM_OK;
}

// ---------------------------------------------------------------------------
// the step
// ---------------------------------------------------------------------------
static hipEvent_t pool_event(lm_model* m) {
    if (m->ev_used == m->ev_pool.size()) {
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        m->ev_pool.push_back(e);
    }
    return m->ev_pool[m->ev_used++];
}

// The node the model's stream would attach the next captured operation to
// (nullptr when nothing has been captured yet); false when not capturing.
static bool capture_tail(lm_model* m, hipGraphNode_t* tail) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipGraphNode_t* deps = nullptr;
    size_t nd = 0;
    if (hipStreamGetCaptureInfo_v2(m->stream, &cs, nullptr, nullptr, &deps, &nd) != hipSuccess ||
        cs != hipStreamCaptureStatusActive)
        return false;
    *tail = nd ? deps[nd - 1] : nullptr;
    return true;
}

// Timing of one kernel family's launches.  Eager (mode 1): HIP events on the
// model's stream around the launches.  Inside a graph capture (mode 2): the
// captured nodes are noted, and event-record nodes are put around them when
// the capture ends (events recorded on a capturing stream are not supported by
// every HIP runtime this library meets).
struct KTimer {
    lm_model* m;
    int kind;
    hipEvent_t a = nullptr;
    bool captured = false;
    hipGraphNode_t before = nullptr;
    KTimer(lm_model* mm, int k) : m(mm), kind(k) {
        if (!m->timing) return;
        if (m->timing == 2 && capture_tail(m, &before)) {
            captured = true;
            return;
        }
        a = pool_event(m);
        if (a && hipEventRecord(a, m->stream) != hipSuccess && m->timer_err == hipSuccess)
            m->timer_err = hipErrorUnknown;
    }
    ~KTimer() {
        if (!m->timing) return;
        if (captured) {
            hipGraphNode_t last = nullptr;
            if (capture_tail(m, &last) && last && last != before) m->cap_scopes.push_back({kind, before, last});
            return;
        }
        if (a) {
            hipEvent_t b = pool_event(m);
            if (b) {
                if (hipEventRecord(b, m->stream) != hipSuccess && m->timer_err == hipSuccess)
                    m->timer_err = hipErrorUnknown;
                m->pending.push_back({kind, a, b});
            }
        }
    }
};

// Puts an event-record node before the first and after the last node of every
// timed scope of a captured (linear) step graph.  Scopes are handled last to
// first, so each one's own edges are still those of the capture.
static hipError_t insert_timers(lm_model* m, hipGraph_t graph, std::vector<lm_model::Pending>& timers,
                                std::vector<hipEvent_t>& owned) {
    hipError_t e = hipSuccess;
    auto deps_of = [](hipGraphNode_t n, std::vector<hipGraphNode_t>& out) {
        size_t nd = 0;
        hipError_t r = hipGraphNodeGetDependencies(n, nullptr, &nd);
        out.resize(nd);
        if (r == hipSuccess && nd) r = hipGraphNodeGetDependencies(n, out.data(), &nd);
        return r;
    };
    auto dependents_of = [](hipGraphNode_t n, std::vector<hipGraphNode_t>& out) {
        size_t nd = 0;
        hipError_t r = hipGraphNodeGetDependentNodes(n, nullptr, &nd);
        out.resize(nd);
        if (r == hipSuccess && nd) r = hipGraphNodeGetDependentNodes(n, out.data(), &nd);
        return r;
    };
    std::vector<lm_model::Pending> found;
    for (size_t i = m->cap_scopes.size(); i-- > 0;) {
        const auto& sc = m->cap_scopes[i];
        // the scope's first node: walk back from its last to the node after `before`
        hipGraphNode_t first = sc.last;
        std::vector<hipGraphNode_t> d;
        for (;;) {
            if ((e = deps_of(first, d)) != hipSuccess) return e;
            if (d.empty() || (d.size() == 1 && d[0] == sc.before)) break;
            if (d.size() != 1) return hipErrorInvalidValue;     // not a linear chain
            first = d[0];
        }
        hipEvent_t ea = nullptr, eb = nullptr;
        if ((e = hipEventCreate(&ea)) != hipSuccess) return e;
        owned.push_back(ea);
        if ((e = hipEventCreate(&eb)) != hipSuccess) return e;
        owned.push_back(eb);
        // after the last node: last -> B -> (what followed last)
        std::vector<hipGraphNode_t> next;
        if ((e = dependents_of(sc.last, next)) != hipSuccess) return e;
        hipGraphNode_t nb = nullptr;
        if ((e = hipGraphAddEventRecordNode(&nb, graph, &sc.last, 1, eb)) != hipSuccess) return e;
        for (hipGraphNode_t n : next) {
            if ((e = hipGraphRemoveDependencies(graph, &sc.last, &n, 1)) != hipSuccess) return e;
            if ((e = hipGraphAddDependencies(graph, &nb, &n, 1)) != hipSuccess) return e;
        }
        // before the first node: (its dependency) -> A -> first
        hipGraphNode_t na = nullptr;
        if ((e = hipGraphAddEventRecordNode(&na, graph, d.empty() ? nullptr : d.data(), d.size(), ea)) != hipSuccess)
            return e;
        for (hipGraphNode_t n : d)
            if ((e = hipGraphRemoveDependencies(graph, &n, &first, 1)) != hipSuccess) return e;
        if ((e = hipGraphAddDependencies(graph, &na, &first, 1)) != hipSuccess) return e;
        found.push_back({sc.kind, ea, eb});
    }
    timers.assign(found.rbegin(), found.rend());
    return hipSuccess;
}

static lm_status collect_timing(lm_model* m) {
    if (m->timer_err != hipSuccess) {
        m->timer_err = hipSuccess;
        m->pending.clear();
        m->ev_used = 0;
        return fail(m, LM_E_HIP, "recording a kernel-timing event failed");
    }
    if (m->pending.empty()) return LM_OK;
    HIPTRY(m, hipStreamSynchronize(m->stream));
    HIPTRY(m, hipStreamSynchronize(m->copy_stream));
    for (auto& p : m->pending) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
            m->kcount[p.kind] += 1;
            m->kms[p.kind] += ms;
        }
    }
    m->pending.clear();
    m->ev_used = 0;
    return LM_OK;
}

// Attention grid of a step: 64-position chunks up to the next multiple of
// four (256 positions) of the longest context among the stepping sequences
// (at most max_chunks), so a launch reads at most three chunks past the
// context (their K/V loads are issued before the position is known).  A step
// graph is keyed by it: a context crossing a multiple of 256 takes a new graph.
static int attn_chunks_for(const lm_model* m, int need) {
    const int tiles = (std::max(need, 1) + kAttnChunk - 1) / kAttnChunk;
    return std::min((tiles + 3) / 4 * 4, m->max_chunks);
}

static int attn_grid_chunks(const lm_model* m, int n_seq) {
    int need = 1;
    for (int s = 0; s < n_seq; ++s) need = std::max(need, m->pos[s] + 1);
    return attn_chunks_for(m, need);
}

static const uint8_t* layer_blob(lm_model* m, int l) {
    return layer_streamed(m, l) ? m->d_sbuf[stream_slot(m, l)] : m->d_layers + (int64_t)l * m->blob_bytes;
}

static lm_status stream_copy(lm_model* m, int layer) {
    const int slot = stream_slot(m, layer);
    HIPTRY(m, hipStreamWaitEvent(m->copy_stream, m->ev_consumed[slot], 0));
    hipEvent_t a = m->timing ? pool_event(m) : nullptr;
    if (a) HIPTRY(m, hipEventRecord(a, m->copy_stream));
    HIPTRY(m, hipMemcpyAsync(m->d_sbuf[slot], host_blob(m, layer), (size_t)m->blob_bytes, hipMemcpyHostToDevice,
                             m->copy_stream));
    if (a) {
        hipEvent_t b = pool_event(m);
        if (b) {
            HIPTRY(m, hipEventRecord(b, m->copy_stream));
            m->pending.push_back({LM_K_COPY, a, b});
        }
    }
    HIPTRY(m, hipEventRecord(m->ev_copied[slot], m->copy_stream));
    return LM_OK;
}

// One sequence: the integer-digit VALU GEMV.  Two to four: activation
// fragments plus the MFMA GEMV (one read of the weights for all sequences).
static hipError_t gemv(lm_model* m, GemvArgs a, int epi, int n_seq, hipStream_t st) {
    if (n_seq >= 2) {
        a.xfrag = m->sb.xfrag;
        return launch_gemv_batched(a, epi, n_seq, m->gemv_max_blocks, st);
    }
    return launch_gemv(a, epi, n_seq, m->gemv_max_blocks, st);
}

// Launch this family's kernels?  All of them, unless a timing-only graph of
// one family is being captured (lm_time_kind).
static bool want(const lm_model* m, int kind) { return m->only_kind < 0 || m->only_kind == kind; }

static lm_status enqueue_step(lm_model* m, int n_seq, const int* d_tok, float* d_logits, int* d_argmax) {
    const lm_config& c = m->cfg;
    const int L = c.n_layers;
    hipStream_t st = m->stream;
    {
        KTimer t(m, LM_K_EMBED);
        if (want(m, LM_K_EMBED)) HIPTRY(m, launch_embed(m->d_embd, d_tok, (int)m->V, (int)m->H, m->sb.x, n_seq, st));
    }
    GemvArgs base{};
    base.qtype = c.qtype;
    base.eps = (float)c.rms_eps;
    base.head_dim = (int)m->hd;
    base.max_ctx = c.max_ctx;
    base.q_rows = (int)m->qrows;
    base.kv_rows = (int)m->kvrows;
    const int* step_pos = m->opt_active && m->opt_pos ? m->opt_pos : m->d_pos;
    const int64_t kv_stride = m->opt_active && m->opt_shared_kv ? 0 : kv_seq_elems(m);
    base.kv_seq_stride = kv_stride;
    base.pos = step_pos;
    base.rope_cos = m->d_cos;
    base.rope_sin = m->d_sin;

    AttnArgs at{};
    at.q = m->sb.q;
    at.kv_seq_stride = kv_stride;
    at.pos = step_pos;
    at.nq = (int)m->nq;
    at.nkv = (int)m->nkv;
    at.hd = (int)m->hd;
    at.max_ctx = c.max_ctx;
    at.max_chunks = m->max_chunks;
    at.scale = (float)(1.0 / std::sqrt((double)m->hd));
    at.grid_chunks = m->opt_active ? attn_chunks_for(m, m->opt_need) : attn_grid_chunks(m, n_seq);
    at.tiles = attn_tiles(n_seq, (int)m->nkv, at.grid_chunks, (int)m->hd);
    at.part = m->sb.attn_part;
    at.counter = m->sb.attn_cnt;
    at.out = m->sb.o;

    const int n_str = (int)m->str_list.size();     // streamed layers this step computes
    const bool serial = m->stream_serial;
    for (int i = 0; i < std::min(n_str, 2) && !serial; ++i)
        if (!m->prefetched[i]) {
            lm_status s = stream_copy(m, m->str_list[i]);
            if (s != LM_OK) return s;
        }
    m->prefetched[0] = m->prefetched[1] = false;

    for (int l = 0; l < L; ++l) {
        if (m->skip[l]) continue;                       // its input is its output
        if (m->opt_active && l >= m->opt_limit) continue;
        if (layer_streamed(m, l) && serial) {
            // everything before this layer has finished, then its copy alone
            HIPTRY(m, hipEventRecord(m->ev_serial, st));
            HIPTRY(m, hipStreamWaitEvent(m->copy_stream, m->ev_serial, 0));
            lm_status s = stream_copy(m, l);
            if (s != LM_OK) return s;
        }
        if (layer_streamed(m, l)) HIPTRY(m, hipStreamWaitEvent(st, m->ev_copied[stream_slot(m, l)], 0));
        if (m->sim_on)                                  // the layer's input, for its similarity
            HIPTRY(m, hipMemcpyAsync(m->d_xin, m->sb.x, (size_t)n_seq * m->H * 4, hipMemcpyDeviceToDevice, st));
        const uint8_t* blob = layer_blob(m, l);
        const float* g_attn = m->d_norms + (int64_t)l * 2 * m->H;
        const float* g_ffn = g_attn + m->H;
        __half* kc = m->d_k + (int64_t)l * kv_layer_elems(m);
        __half* vc = m->d_v + (int64_t)l * kv_layer_elems(m);
        {   // RMSNorm -> QKV GEMV -> RoPE -> KV append
            KTimer t(m, LM_K_QKV);
            GemvArgs a = base;
            a.w = mat_at(m, blob, M_QKV);
            a.xin = m->sb.x; a.x_stride = (int)m->H;
            a.norm_g = g_attn;
            a.out = m->sb.q; a.out_stride = (int)m->qrows;
            a.kcache = kc; a.vcache = vc;
            if (want(m, LM_K_QKV)) HIPTRY(m, gemv(m, a, EPI_QKV, n_seq, st));
        }
        {   // GQA attention with causal softmax
            KTimer t(m, LM_K_ATTN);
            AttnArgs b = at;
            b.kcache = kc; b.vcache = vc;
            if (want(m, LM_K_ATTN)) HIPTRY(m, launch_attention(b, n_seq, st));
        }
        {   // x += Wo o
            KTimer t(m, LM_K_WO);
            GemvArgs a = base;
            a.w = mat_at(m, blob, M_WO);
            a.xin = m->sb.o; a.x_stride = (int)m->qrows;
            a.out = m->sb.x; a.out_stride = (int)m->H;
            if (want(m, LM_K_WO)) HIPTRY(m, gemv(m, a, EPI_RESID, n_seq, st));
        }
        {   // RMSNorm -> gate/up GEMV -> SwiGLU
            KTimer t(m, LM_K_GATEUP);
            GemvArgs a = base;
            a.w = mat_at(m, blob, M_GU);
            a.xin = m->sb.x; a.x_stride = (int)m->H;
            a.norm_g = g_ffn;
            a.out = m->sb.h; a.out_stride = (int)m->F;
            if (want(m, LM_K_GATEUP)) HIPTRY(m, gemv(m, a, EPI_SWIGLU, n_seq, st));
        }
        {   // x += Wdown h
            KTimer t(m, LM_K_DOWN);
            GemvArgs a = base;
            a.w = mat_at(m, blob, M_DOWN);
            a.xin = m->sb.h; a.x_stride = (int)m->F;
            a.out = m->sb.x; a.out_stride = (int)m->H;
            a.xfrag_ready = n_seq >= 2 && gateup_writes_digits(m->F);   // h's digits came with h
            if (want(m, LM_K_DOWN)) HIPTRY(m, gemv(m, a, EPI_RESID, n_seq, st));
        }
        if (m->sim_on) HIPTRY(m, launch_layer_cos(m->d_xin, m->sb.x, (int)m->H, n_seq, m->d_sim + 2 * l, st));
        if (layer_streamed(m, l)) {
            HIPTRY(m, hipEventRecord(m->ev_consumed[stream_slot(m, l)], st));
            const int nx = m->str_idx[l] + 2;
            if (nx < n_str && !serial) {
                lm_status s = stream_copy(m, m->str_list[nx]);
                if (s != LM_OK) return s;
            }
        }
    }
    // start the next step's first two streamed layers while the LM head (and
    // the next step's resident layers) run
    for (int i = 0; i < std::min(n_str, 2) && !serial; ++i) {
        lm_status s = stream_copy(m, m->str_list[i]);
        if (s != LM_OK) return s;
        m->prefetched[i] = true;
    }
    {   // final RMSNorm -> LM head GEMV -> argmax (and positions += 1)
        KTimer t(m, LM_K_LMHEAD);
        GemvArgs a = base;
        a.w = lm_head_mat(m);
        a.xin = m->sb.x; a.x_stride = (int)m->H;
        a.norm_g = m->d_out_norm;
        a.out = d_logits; a.out_stride = (int)m->V;
        a.part_val = m->sb.lm_pval;
        a.part_idx = m->sb.lm_pidx;
        a.counter = m->sb.lm_cnt;
        a.argmax_out = d_argmax;
        // a timing-only replay of the LM head must not advance the positions
        a.pos_inc = m->only_kind < 0 && !(m->opt_active && !m->opt_advance) ? m->d_pos : nullptr;
        if (want(m, LM_K_LMHEAD)) HIPTRY(m, gemv(m, a, EPI_LOGITS, n_seq, st));
    }
    return LM_OK;
}

// Launch a captured step; with timers (timing mode 2) wait for it and add the
// durations of the event pairs recorded inside the graph.
static lm_status launch_graph(lm_model* m, const lm_model::GraphEntry& g) {
    HIPTRY(m, hipGraphLaunch(g.exec, m->stream));
    if (g.timers.empty()) return LM_OK;
    for (const auto& t : g.timers) m->pending.push_back(t);
    return collect_timing(m);
}

static lm_status run_step(lm_model* m, int n_seq, const int* d_tok, float* d_logits, int* d_argmax) {
    const bool graph_ok = m->use_graph && m->timing != 1 && !m->streaming && !m->sim_on;
    if (!graph_ok) return enqueue_step(m, n_seq, d_tok, d_logits, d_argmax);
    const int chunks = attn_grid_chunks(m, n_seq);
    for (auto& g : m->graphs)
        if (g.n_seq == n_seq && g.chunks == chunks && g.tok == d_tok && g.logits == d_logits &&
            g.argmax == d_argmax)
            return launch_graph(m, g);
    lm_status cs = collect_timing(m);
    if (cs != LM_OK) return cs;
    m->cap_scopes.clear();
    hipGraph_t graph = nullptr;
    HIPTRY(m, hipStreamBeginCapture(m->stream, hipStreamCaptureModeThreadLocal));
    lm_status s = enqueue_step(m, n_seq, d_tok, d_logits, d_argmax);
    hipError_t e = hipStreamEndCapture(m->stream, &graph);
    std::vector<lm_model::Pending> timers;
    std::vector<hipEvent_t> owned;
    if (s == LM_OK && e == hipSuccess && m->timing == 2) {
        const hipError_t te = insert_timers(m, graph, timers, owned);
        if (te != hipSuccess)
            s = fail(m, LM_E_HIP, "placing timing events in the step graph failed: %s", hipGetErrorString(te));
    }
    m->cap_scopes.clear();
    if (s != LM_OK || e != hipSuccess) {
        if (graph) (void)hipGraphDestroy(graph);
        for (hipEvent_t ev : owned) (void)hipEventDestroy(ev);
        if (s != LM_OK) return s;
        return fail(m, LM_E_HIP, "hipStreamEndCapture failed: %s", hipGetErrorString(e));
    }
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) {
        for (hipEvent_t ev : owned) (void)hipEventDestroy(ev);
        return fail(m, LM_E_HIP, "hipGraphInstantiate failed: %s", hipGetErrorString(e));
    }
    if (m->graphs.size() >= 8) {
        (void)hipGraphExecDestroy(m->graphs.front().exec);
        for (hipEvent_t ev : m->graphs.front().owned) (void)hipEventDestroy(ev);
        m->graphs.erase(m->graphs.begin());
    }
    m->graphs.push_back({n_seq, chunks, d_tok, d_logits, d_argmax, exec, std::move(timers), std::move(owned)});
    return launch_graph(m, m->graphs.back());
}

static lm_status check_ready(lm_model* m, const char* fn, int n_seq) {
    if (!m->global_loaded)
        return fail(m, LM_E_STATE, "%s: global weights not loaded (lm_load_global_weights)", fn);
    for (int l = 0; l < m->cfg.n_layers; ++l)
        if (!m->layer_loaded[l]) return fail(m, LM_E_STATE, "%s: layer %d weights not loaded", fn, l);
    if (n_seq < 1 || n_seq > m->cfg.max_seqs)
        return fail(m, LM_E_ARG, "%s: n_seq = %d; expected 1..%d (max_seqs)", fn, n_seq, m->cfg.max_seqs);
    for (int s = 0; s < n_seq; ++s)
        if (m->pos[s] + 1 > m->cfg.max_ctx)
            return fail(m, LM_E_CTX, "%s: sequence %d is at position %d; max_ctx = %d leaves no room for a step",
                        fn, s, m->pos[s], m->cfg.max_ctx);
    return LM_OK;
}

extern "C" lm_status lm_decode_step(lm_model* m, const int32_t* tokens, int32_t n_seq, float* logits,
                                    int32_t* argmax) {
    if (!m) return LM_E_ARG;
    lm_status st = check_ready(m, "lm_decode_step", n_seq);
    if (st != LM_OK) return st;
    if (!tokens || !argmax) return fail(m, LM_E_ARG, "lm_decode_step: tokens or argmax is NULL");
    for (int s = 0; s < n_seq; ++s)
        if (tokens[s] < 0 || tokens[s] >= m->cfg.vocab)
            return fail(m, LM_E_ARG, "lm_decode_step: tokens[%d] = %d; expected 0..%d", s, tokens[s],
                        m->cfg.vocab - 1);
    HIPTRY(m, hipMemcpyAsync(m->d_tokens, tokens, (size_t)n_seq * 4, hipMemcpyHostToDevice, m->stream));
    st = run_step(m, n_seq, m->d_tokens, logits ? m->d_logits : nullptr, m->d_argmax);
    if (st != LM_OK) return st;
    for (int s = 0; s < n_seq; ++s) m->pos[s] += 1;
    HIPTRY(m, hipMemcpyAsync(argmax, m->d_argmax, (size_t)n_seq * 4, hipMemcpyDeviceToHost, m->stream));
    if (logits)
        HIPTRY(m, hipMemcpyAsync(logits, m->d_logits, (size_t)(n_seq * m->V * 4), hipMemcpyDeviceToHost,
                                 m->stream));
    HIPTRY(m, hipStreamSynchronize(m->stream));
    return collect_timing(m);
}

extern "C" lm_status lm_decode_step_dev(lm_model* m, const int32_t* d_tokens, int32_t n_seq, float* d_logits,
                                        int32_t* d_argmax) {
    if (!m) return LM_E_ARG;
    lm_status st = check_ready(m, "lm_decode_step_dev", n_seq);
    if (st != LM_OK) return st;
    if (!d_tokens || !d_argmax) return fail(m, LM_E_ARG, "lm_decode_step_dev: d_tokens or d_argmax is NULL");
    st = run_step(m, n_seq, d_tokens, d_logits, d_argmax);
    if (st != LM_OK) return st;
    for (int s = 0; s < n_seq; ++s) m->pos[s] += 1;
    return LM_OK;
}

// The step's working buffers for n_seq sequences as slices of one region at
// base, each 256-byte aligned; returns the bytes they need (base == nullptr:
// the size only).  The counts and the activation digits come first, so that
// one clear covers what must start at zero: [0, *zero_bytes).
static int64_t scratch_layout(const lm_model* m, int n_seq, uint8_t* base, StepBufs* b, int64_t* zero_bytes) {
    int64_t off = 0;
    auto take = [&](int64_t bytes) {
        uint8_t* p = base ? base + off : nullptr;
        off += (bytes + 255) / 256 * 256;
        return p;
    };
    const int64_t S = n_seq;
    StepBufs t;
    t.attn_cnt = (int*)take(S * m->nkv * attn_cnt_lines(m->max_chunks) * kCntStride * 4);
    t.lm_cnt = (int*)take(S * 4);
    if (m->batched && n_seq >= 2) t.xfrag = take(xfrag_bytes(std::max<int64_t>({m->H, m->qrows, m->F})));
    const int64_t zeroed = off;
    t.x = (float*)take(S * m->H * 4);
    t.q = (float*)take(S * m->qrows * 4);
    t.o = (float*)take(S * m->qrows * 4);
    t.h = (float*)take(S * m->F * 4);
    t.attn_part = (float*)take(S * m->nq * m->max_chunks * (m->hd + 2) * 4);
    t.lm_pval = (float*)take(S * m->gemv_max_blocks * 4);
    t.lm_pidx = (int*)take(S * m->gemv_max_blocks * 4);
    if (b) *b = t;
    if (zero_bytes) *zero_bytes = zeroed;
    return off;
}

extern "C" lm_status lm_decode_step_dev_noalloc(lm_model* m, const int32_t* d_tokens, int32_t n_seq,
                                                float* d_logits, int32_t* d_argmax) {
    if (!m) return LM_E_ARG;
    lm_status st = check_ready(m, "lm_decode_step_dev_noalloc", n_seq);
    if (st != LM_OK) return st;
    if (!d_tokens || !d_argmax)
        return fail(m, LM_E_ARG, "lm_decode_step_dev_noalloc: d_tokens or d_argmax is NULL");
    if (m->streaming)
        return fail(m, LM_E_STATE, "lm_decode_step_dev_noalloc: layers %d..%d are streamed; every layer must be "
                    "resident (lm_set_residency with n_layers)", m->n_res, m->cfg.n_layers - 1);
    const int64_t need = scratch_layout(m, n_seq, nullptr, nullptr, nullptr);
    if (need > kNoAllocScratchBytes)
        return fail(m, LM_E_ARG, "lm_decode_step_dev_noalloc: %d sequences with max_ctx %d need %lld bytes of "
                    "scratch; the allocation-free step has %lld (use lm_decode_step_dev)", n_seq, m->cfg.max_ctx,
                    (long long)need, (long long)kNoAllocScratchBytes);
    uint8_t* base = nullptr;
    const hipError_t e = noalloc_scratch(m->device, &base);
    if (e != hipSuccess)
        return fail(m, LM_E_HIP, "lm_decode_step_dev_noalloc: scratch address: %s", hipGetErrorString(e));
    StepBufs sb;
    int64_t zero_bytes = 0;
    scratch_layout(m, n_seq, base, &sb, &zero_bytes);
    // the array keeps the last call's contents (possibly another model's)
    HIPTRY(m, launch_zero(base, zero_bytes, m->stream));
    // eager launches (instantiating a graph would allocate), no timing events
    const StepBufs own = m->sb;
    const int timing = m->timing;
    m->sb = sb;
    m->timing = 0;
    st = enqueue_step(m, n_seq, d_tokens, d_logits, d_argmax);
    m->sb = own;
    m->timing = timing;
    if (st != LM_OK) return st;
    for (int s = 0; s < n_seq; ++s) m->pos[s] += 1;
    return LM_OK;
}

// ---------------------------------------------------------------------------
// self-speculative decoding (the C/CUDA Llama engine page, sections 3.5, 5.3)
// ---------------------------------------------------------------------------
// One round for sequence 0: k drafts, each one step of the layers below
// draft_layers and the LM head; then one pass of the whole model over the k+1
// tokens t0, d1..dk at positions p..p+k as k+1 columns of the several-sequence
// path that all read and write sequence 0's cache (column j attends to keys
// 0..p+j, the block's own keys included: the verify pass is exactly k+1 plain
// steps); then the longest prefix of drafts that the full model agrees with,
// plus the full model's token after it.
extern "C" lm_status lm_speculative_step(lm_model* m, int32_t token, int32_t draft_layers, int32_t k,
                                         int32_t* tokens_out, int32_t* n_out) {
    if (!m) return LM_E_ARG;
    lm_status st = check_ready(m, "lm_speculative_step", 1);
    if (st != LM_OK) return st;
    const int L = m->cfg.n_layers;
    if (!tokens_out || !n_out) return fail(m, LM_E_ARG, "lm_speculative_step: tokens_out or n_out is NULL");
    if (m->cfg.max_seqs < 2)
        return fail(m, LM_E_STATE, "lm_speculative_step: the verify pass runs k + 1 tokens as sequences of the "
                    "several-sequence path; max_seqs = %d; expected 2..4 (Q8_0 / Q4_0 models)", m->cfg.max_seqs);
    if (k < 1 || k > 3 || k + 1 > m->cfg.max_seqs)
        return fail(m, LM_E_ARG, "lm_speculative_step: k = %d; expected 1..%d (k + 1 <= max_seqs <= 4)", k,
                    std::min(3, m->cfg.max_seqs - 1));
    if (draft_layers < 0 || draft_layers > L)
        return fail(m, LM_E_ARG, "lm_speculative_step: draft_layers = %d; expected 0..%d", draft_layers, L);
    if (token < 0 || token >= m->cfg.vocab)
        return fail(m, LM_E_ARG, "lm_speculative_step: token = %d; expected 0..%d", token, m->cfg.vocab - 1);
    if (m->streaming)
        return fail(m, LM_E_STATE, "lm_speculative_step: not in streaming mode (every layer must be resident)");
    const int p = m->pos[0];
    if (p + k + 1 > m->cfg.max_ctx)
        return fail(m, LM_E_CTX, "lm_speculative_step: position %d + %d drafts reaches max_ctx = %d", p, k,
                    m->cfg.max_ctx);
    hipStream_t s0 = m->stream;
    HIPTRY(m, hipMemcpyAsync(m->d_spec, &token, 4, hipMemcpyHostToDevice, s0));
    // drafts: the bottom layers, positions advanced on the device as a plain step does
    m->opt_active = true;
    m->opt_pos = nullptr;
    m->opt_shared_kv = false;
    m->opt_advance = true;
    m->opt_limit = draft_layers;
    for (int i = 0; i < k && st == LM_OK; ++i) {
        m->opt_need = p + i + 1;
        st = enqueue_step(m, 1, m->d_spec + i, nullptr, m->d_spec + i + 1);
        if (st == LM_OK) m->pos[0] += 1;
    }
    // verify: every layer, columns j = 0..k at positions p + j on sequence 0's cache
    int32_t vpos[4] = {p, p + 1, p + 2, p + 3};
    int32_t h[16] = {0};
    if (st == LM_OK) {
        const hipError_t e = hipMemcpyAsync(m->d_vpos, vpos, 16, hipMemcpyHostToDevice, s0);
        if (e != hipSuccess) st = fail(m, LM_E_HIP, "lm_speculative_step: %s", hipGetErrorString(e));
    }
    if (st == LM_OK) {
        m->opt_pos = m->d_vpos;
        m->opt_shared_kv = true;
        m->opt_advance = false;
        m->opt_limit = L;
        m->opt_need = p + k + 1;
        st = enqueue_step(m, k + 1, m->d_spec, nullptr, m->d_spec + 8);
    }
    m->opt_active = false;
    m->opt_pos = nullptr;
    if (st != LM_OK) return st;
    HIPTRY(m, hipMemcpyAsync(h, m->d_spec, sizeof(h), hipMemcpyDeviceToHost, s0));
    HIPTRY(m, hipStreamSynchronize(s0));
    // the longest agreeing prefix of drafts, then the full model's own token
    int n = 0;
    while (n < k && h[8 + n] == h[1 + n]) {
        tokens_out[n] = h[1 + n];
        ++n;
    }
    tokens_out[n] = h[8 + n];
    *n_out = n + 1;
    m->pos[0] = p + n + 1;
    HIPTRY(m, hipMemcpy(m->d_pos, &m->pos[0], 4, hipMemcpyHostToDevice));
    return collect_timing(m);
}

extern "C" lm_status lm_set_graph(lm_model* m, int32_t enable) {
    if (!m) return LM_E_ARG;
    m->use_graph = enable != 0;
    if (!m->use_graph) {
        HIPTRY(m, hipStreamSynchronize(m->stream));
        invalidate_graphs(m);
    }
    return LM_OK;
}

// ---------------------------------------------------------------------------
// streaming mode
// ---------------------------------------------------------------------------
// The C/CUDA Llama engine page's tier sizing (its section 4.1): tier A (HBM)
// takes floor(0.9 * free HBM / layer bytes) layers, tier B (pinned host
// memory) floor(0.7 * available host memory / layer bytes); what fits in
// neither would go to a disk tier, which this library does not have.
extern "C" lm_status lm_tier_sizes(int32_t n_layers, int64_t layer_bytes, int64_t hbm_bytes, int64_t host_bytes,
                                   int32_t* tier_a, int32_t* tier_b) {
    if (n_layers < 1 || layer_bytes < 1 || hbm_bytes < 0 || host_bytes < 0 || !tier_a || !tier_b) return LM_E_ARG;
    // exact floors of 0.9 * hbm / layer and 0.7 * host / layer
    const __int128 den = (__int128)10 * layer_bytes;
    const int64_t a = (int64_t)std::min<__int128>(n_layers, (__int128)9 * hbm_bytes / den);
    const int64_t b = (int64_t)std::min<__int128>(n_layers - a, (__int128)7 * host_bytes / den);
    *tier_a = (int32_t)a;
    *tier_b = (int32_t)b;
    return a + b == n_layers ? LM_OK : LM_E_OOM;
}

extern "C" lm_status lm_plan_residency(lm_model* m, int64_t hbm_bytes, int64_t host_bytes, int32_t* n_resident) {
    if (!m || !n_resident) return LM_E_ARG;
    if (hbm_bytes <= 0) {
        size_t fr = 0, tot = 0;
        HIPTRY(m, hipMemGetInfo(&fr, &tot));
        // the resident layers' own bytes would be free too
        hbm_bytes = (int64_t)fr + (int64_t)m->n_res * m->blob_bytes;
    }
    if (host_bytes <= 0) {
        const long pages = sysconf(_SC_AVPHYS_PAGES), psz = sysconf(_SC_PAGESIZE);
        host_bytes = (pages > 0 && psz > 0 ? (int64_t)pages * psz : 0) +
                    (int64_t)(m->cfg.n_layers - m->n_res) * m->blob_bytes;
    }
    int32_t a = 0, b = 0;
    const lm_status st = lm_tier_sizes(m->cfg.n_layers, m->blob_bytes, hbm_bytes, host_bytes, &a, &b);
    *n_resident = a;
    if (st != LM_OK)
        return fail(m, st, "lm_plan_residency: %d resident + %d host layers of %d fit (HBM %lld B, host %lld B)",
                    a, b, m->cfg.n_layers, (long long)hbm_bytes, (long long)host_bytes);
    return LM_OK;
}

extern "C" lm_status lm_set_residency(lm_model* m, int32_t n_resident) {
    if (!m) return LM_E_ARG;
    const int L = m->cfg.n_layers;
    if (n_resident < 0 || n_resident > L)
        return fail(m, LM_E_ARG, "lm_set_residency: n_resident = %d; expected 0..%d", n_resident, L);
    if (n_resident == m->n_res) {
        m->stream_serial = false;               // (serial streaming only through lm_stream_mode 2)
        return LM_OK;
    }
    HIPTRY(m, hipStreamSynchronize(m->stream));
    HIPTRY(m, hipStreamSynchronize(m->copy_stream));
    const int64_t B = m->blob_bytes;
    const int old = m->n_res, nw = n_resident;
    uint8_t *d = nullptr, *h = nullptr, *b0 = m->d_sbuf[0], *b1 = m->d_sbuf[1];
    const bool new_bufs = nw < L && !b0;
    // The layers that stay streamed keep their place in the present pinned
    // arena when it can hold the new set: more layers resident (the front of
    // the allocation is left unused), or fewer when that unused front is large
    // enough for the layers coming back.  Otherwise a new arena is allocated
    // before the old one is freed.
    const bool keep_arena = m->h_arena && nw < L &&
                            (nw > old || (int64_t)(m->h_arena - m->h_arena_alloc) >= (int64_t)(old - nw) * B);
    lm_status st = LM_OK;
    if (nw > 0) st = dev_alloc(m, (void**)&d, nw * B, "layer weights");
    if (st == LM_OK && nw < L) {
        if (keep_arena) h = m->h_arena + (int64_t)(nw - old) * B;
        else st = host_alloc(m, (void**)&h, (L - nw) * B, "streaming host arena");
    }
    if (st == LM_OK && new_bufs) {
        b0 = b1 = nullptr;
        st = dev_alloc(m, (void**)&b0, B, "streaming buffer 0");
        if (st == LM_OK) st = dev_alloc(m, (void**)&b1, B, "streaming buffer 1");
    }
    // every layer from its present home to its new one
    for (int l = 0; l < L && st == LM_OK; ++l) {
        const bool from_dev = l < old, to_dev = l < nw;
        const uint8_t* src = from_dev ? m->d_layers + (int64_t)l * B : m->h_arena + (int64_t)(l - old) * B;
        uint8_t* dst = to_dev ? d + (int64_t)l * B : h + (int64_t)(l - nw) * B;
        if (!from_dev && !to_dev) {
            if (dst != src) std::memcpy(dst, src, (size_t)B);
            continue;
        }
        const hipMemcpyKind kind = from_dev ? (to_dev ? hipMemcpyDeviceToDevice : hipMemcpyDeviceToHost)
                                            : hipMemcpyHostToDevice;
        const hipError_t e = hipMemcpy(dst, src, (size_t)B, kind);
        if (e != hipSuccess)
            st = fail(m, LM_E_HIP, "lm_set_residency: moving layer %d failed: %s", l, hipGetErrorString(e));
    }
    if (st != LM_OK) {
        dev_free(m, d);
        if (!keep_arena) host_free(m, h);
        if (new_bufs) {
            dev_free(m, b0);
            dev_free(m, b1);
        }
        return st;
    }
    dev_free(m, m->d_layers);
    if (!keep_arena) {
        host_free(m, m->h_arena_alloc);
        m->h_arena_alloc = nw < L ? h : nullptr;
    }
    if (nw == L) {
        dev_free(m, b0);
        dev_free(m, b1);
        b0 = b1 = nullptr;
    }
    m->d_layers = d;
    m->h_arena = h;
    m->d_sbuf[0] = b0;
    m->d_sbuf[1] = b1;
    m->n_res = nw;
    m->streaming = nw < L;
    rebuild_stream_order(m);
    m->prefetched[0] = m->prefetched[1] = false;
    invalidate_graphs(m);
    m->stream_serial = false;
    return LM_OK;
}

// ---------------------------------------------------------------------------
// layer skip (the C/CUDA Llama engine page, sections 2.5, 3.5, 4.5)
// ---------------------------------------------------------------------------
extern "C" lm_status lm_set_layer_skip(lm_model* m, const uint8_t* mask) {
    if (!m) return LM_E_ARG;
    HIPTRY(m, hipStreamSynchronize(m->stream));
    HIPTRY(m, hipStreamSynchronize(m->copy_stream));
    const int L = m->cfg.n_layers;
    m->any_skip = false;
    for (int l = 0; l < L; ++l) {
        m->skip[l] = mask && mask[l] ? 1 : 0;
        m->any_skip = m->any_skip || m->skip[l];
    }
    rebuild_stream_order(m);
    m->prefetched[0] = m->prefetched[1] = false;
    invalidate_graphs(m);
    return LM_OK;
}

extern "C" lm_status lm_layer_similarity(lm_model* m, int32_t enable) {
    if (!m) return LM_E_ARG;
    HIPTRY(m, hipStreamSynchronize(m->stream));
    if (enable) HIPTRY(m, hipMemset(m->d_sim, 0, (size_t)m->cfg.n_layers * 2 * 8));
    m->sim_on = enable != 0;
    invalidate_graphs(m);
    return LM_OK;
}

extern "C" lm_status lm_get_layer_similarity(lm_model* m, double* mean, int32_t* count) {
    if (!m || !mean) return LM_E_ARG;
    const int L = m->cfg.n_layers;
    std::vector<double> h((size_t)L * 2);
    HIPTRY(m, hipStreamSynchronize(m->stream));
    HIPTRY(m, hipMemcpy(h.data(), m->d_sim, h.size() * 8, hipMemcpyDeviceToHost));
    for (int l = 0; l < L; ++l) {
        mean[l] = h[2 * l + 1] > 0 ? h[2 * l] / h[2 * l + 1] : std::nan("");
        if (count) count[l] = (int32_t)h[2 * l + 1];
    }
    return LM_OK;
}

extern "C" lm_status lm_skip_similar_layers(lm_model* m, double threshold, int32_t* n_skipped) {
    if (!m || !std::isfinite(threshold)) return LM_E_ARG;
    const int L = m->cfg.n_layers;
    std::vector<double> mean((size_t)L);
    lm_status st = lm_get_layer_similarity(m, mean.data(), nullptr);
    if (st != LM_OK) return st;
    std::vector<uint8_t> mask((size_t)L);
    int n = 0;
    for (int l = 0; l < L; ++l) {
        mask[l] = mean[l] > threshold;            // false for a layer with no record (NaN)
        n += mask[l];
    }
    if (n_skipped) *n_skipped = n;
    return lm_set_layer_skip(m, mask.data());
}

extern "C" lm_status lm_stream_mode(lm_model* m, int32_t enable) {
    if (!m) return LM_E_ARG;
    if (enable < 0 || enable > 2) return fail(m, LM_E_ARG, "lm_stream_mode: mode = %d; expected 0, 1 or 2", enable);
    lm_status st = lm_set_residency(m, enable ? 0 : m->cfg.n_layers);
    if (st != LM_OK) return st;
    HIPTRY(m, hipStreamSynchronize(m->stream));
    HIPTRY(m, hipStreamSynchronize(m->copy_stream));
    // nothing is left copied ahead of a step, whichever mode follows
    m->prefetched[0] = m->prefetched[1] = false;
    m->stream_serial = enable == 2;
    return LM_OK;
}

// ---------------------------------------------------------------------------
// measurement and inspection
// ---------------------------------------------------------------------------
extern "C" lm_status lm_kernel_timing(lm_model* m, int32_t enable) {
    if (!m) return LM_E_ARG;
    lm_status st = collect_timing(m);
    if (st != LM_OK) return st;
    if (enable < 0 || enable > 2) return fail(m, LM_E_ARG, "lm_kernel_timing: mode = %d; expected 0, 1 or 2", enable);
    if (enable != m->timing) {
        // graphs captured with (or without) timing events do not serve the other mode
        HIPTRY(m, hipStreamSynchronize(m->stream));
        invalidate_graphs(m);
    }
    m->timing = enable;
    for (int k = 0; k < LM_K_COUNT; ++k) { m->kcount[k] = 0; m->kms[k] = 0.0; }
    return LM_OK;
}

extern "C" lm_status lm_time_kind(lm_model* m, int32_t kind, int32_t n_seq, int32_t reps, double* us_per_launch) {
    if (!m || !us_per_launch || kind < 0 || kind >= LM_K_COUNT || kind == LM_K_COPY || reps < 1) return LM_E_ARG;
    lm_status st = check_ready(m, "lm_time_kind", n_seq);
    if (st != LM_OK) return st;
    if (m->streaming) return fail(m, LM_E_STATE, "lm_time_kind: not in streaming mode (steps there are not graphs)");
    // the step's launches of this family alone, captured as one graph (same
    // arguments and order as in the step), replayed between two events
    HIPTRY(m, hipStreamSynchronize(m->stream));
    const int saved_timing = m->timing;
    m->timing = 0;
    m->only_kind = kind;
    // a family launched once per step is captured 32 times over, so that one
    // graph launch's own cost is spread as thinly as over a per-layer family
    const bool once = kind == LM_K_EMBED || kind == LM_K_LMHEAD;
    const int inner = once ? 32 : 1;
    hipGraph_t graph = nullptr;
    hipError_t e = hipStreamBeginCapture(m->stream, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
        for (int i = 0; i < inner && st == LM_OK; ++i)
            st = enqueue_step(m, n_seq, m->d_tokens, nullptr, m->d_argmax);
        e = hipStreamEndCapture(m->stream, &graph);
    }
    m->only_kind = -1;
    m->timing = saved_timing;
    if (st != LM_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return st;
    }
    if (e != hipSuccess) return fail(m, LM_E_HIP, "lm_time_kind: capture failed: %s", hipGetErrorString(e));
    size_t n_nodes = 0;
    (void)hipGraphGetNodes(graph, nullptr, &n_nodes);
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return fail(m, LM_E_HIP, "lm_time_kind: instantiate failed: %s", hipGetErrorString(e));
    if (n_nodes == 0) {
        (void)hipGraphExecDestroy(exec);
        return fail(m, LM_E_STATE, "lm_time_kind: kind %d launches nothing in this model's step", kind);
    }
    hipEvent_t a = nullptr, b = nullptr;
    float ms = 0.f;
    e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    if (e == hipSuccess) e = hipGraphLaunch(exec, m->stream);          // warm
    if (e == hipSuccess) e = hipEventRecord(a, m->stream);
    for (int r = 0; r < reps && e == hipSuccess; ++r) e = hipGraphLaunch(exec, m->stream);
    if (e == hipSuccess) e = hipEventRecord(b, m->stream);
    if (e == hipSuccess) e = hipEventSynchronize(b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    (void)hipGraphExecDestroy(exec);
    if (e != hipSuccess) return fail(m, LM_E_HIP, "lm_time_kind: %s", hipGetErrorString(e));
    // launches of the family per step (a launch may be more than one graph node:
    // the several-sequence GEMV stages its activations first)
    const double launches = once ? (double)inner : (double)m->cfg.n_layers;
    *us_per_launch = 1e3 * (double)ms / ((double)reps * launches);
    return LM_OK;
}

extern "C" lm_status lm_kernel_stats(lm_model* m, int32_t kind, int64_t* count, double* total_ms) {
    if (!m || kind < 0 || kind >= LM_K_COUNT || !count || !total_ms) return LM_E_ARG;
    lm_status st = collect_timing(m);
    if (st != LM_OK) return st;
    *count = m->kcount[kind];
    *total_ms = m->kms[kind];
    return LM_OK;
}

extern "C" lm_status lm_kernel_bytes(const lm_model* m, int32_t kind, int32_t n_seq, double* bytes) {
    if (!m || !bytes || kind < 0 || kind >= LM_K_COUNT || n_seq < 1 || n_seq > m->cfg.max_seqs) return LM_E_ARG;
    const double bpw = (double)gguf_row_bytes(m->cfg.qtype, 256) / 256.0;   // bytes per weight
    int computed = 0;                                 // layers a step computes (not skipped)
    for (int l = 0; l < m->cfg.n_layers; ++l) computed += !m->skip[l];
    const double H = (double)m->H, F = (double)m->F, V = (double)m->V, Q = (double)m->qrows,
                 KV = (double)m->kvrows, L = computed, S = n_seq;
    double b = 0.0;
    switch (kind) {
        case LM_K_EMBED: b = S * H * (2 + 4); break;
        case LM_K_QKV: b = L * ((Q + 2 * KV) * H * bpw + H * 4 + S * (H * 4 + Q * 4 + 2 * KV * 2)); break;
        case LM_K_ATTN: {
            double kv = 0.0;
            for (int s = 0; s < n_seq; ++s) kv += (double)(m->pos[s] + 1) * KV * 2 * 2;
            b = L * (kv + S * Q * 4 * 2);
            break;
        }
        case LM_K_WO: b = L * (H * Q * bpw + S * (Q * 4 + H * 8)); break;
        case LM_K_GATEUP: b = L * (2 * F * H * bpw + H * 4 + S * (H * 4 + F * 4)); break;
        case LM_K_DOWN: b = L * (H * F * bpw + S * (F * 4 + H * 8)); break;
        case LM_K_LMHEAD: b = V * H * bpw + H * 4 + S * H * 4; break;
        case LM_K_COPY: b = (double)m->str_list.size() * (double)m->blob_bytes; break;
    }
    *bytes = b;
    return LM_OK;
}

extern "C" lm_status lm_debug_dequant(lm_model* m, int32_t layer, int32_t which, int32_t row0, int32_t n_rows,
                                      float* out) {
    if (!m || !out) return LM_E_ARG;
    if (which < 0 || which > 7) return fail(m, LM_E_ARG, "lm_debug_dequant: which = %d; expected 0..7", which);
    if (which < 7 && (layer < 0 || layer >= m->cfg.n_layers))
        return fail(m, LM_E_ARG, "lm_debug_dequant: layer = %d; expected 0..%d", layer, m->cfg.n_layers - 1);
    // (matrix, first device row, row stride, rows available)
    int mat = -1;
    int64_t dr0 = 0, stride = 1, avail = 0;
    switch (which) {
        case 0: mat = M_QKV; dr0 = 0; avail = m->qrows; break;
        case 1: mat = M_QKV; dr0 = m->qrows; avail = m->kvrows; break;
        case 2: mat = M_QKV; dr0 = m->qrows + m->kvrows; avail = m->kvrows; break;
        case 3: mat = M_WO; avail = m->H; break;
        case 4: mat = M_GU; dr0 = 0; stride = 2; avail = m->F; break;
        case 5: mat = M_GU; dr0 = 1; stride = 2; avail = m->F; break;
        case 6: mat = M_DOWN; avail = m->H; break;
        default: avail = m->V; break;
    }
    if (row0 < 0 || n_rows < 0 || row0 + (int64_t)n_rows > avail)
        return fail(m, LM_E_ARG, "lm_debug_dequant: rows [%d, %d) outside 0..%lld", row0, row0 + n_rows,
                    (long long)avail);
    HIPTRY(m, hipStreamSynchronize(m->stream));
    HIPTRY(m, hipStreamSynchronize(m->copy_stream));
    QMat w;
    if (mat < 0) w = lm_head_mat(m);
    else if (layer_streamed(m, layer)) {
        HIPTRY(m, hipMemcpy(m->d_sbuf[0], host_blob(m, layer), (size_t)m->blob_bytes, hipMemcpyHostToDevice));
        m->prefetched[0] = m->prefetched[1] = false;
        w = mat_at(m, m->d_sbuf[0], mat);
    } else {
        w = mat_at(m, m->d_layers + (int64_t)layer * m->blob_bytes, mat);
    }
    const int K = w.K;
    const int64_t per = std::max<int64_t>(1, m->dbg_floats / K);
    std::vector<float> tmp;
    for (int64_t r = 0; r < n_rows;) {
        // device rows for logical rows r.. (stride 1 or 2)
        const int64_t n = std::min<int64_t>(n_rows - r, per / stride);
        const int64_t first = dr0 + (row0 + r) * stride;
        const int64_t span = (n - 1) * stride + 1;
        HIPTRY(m, launch_dequant(w, m->cfg.qtype, (int)first, (int)span, m->d_dbg, m->stream));
        tmp.resize((size_t)(span * K));
        HIPTRY(m, hipMemcpyAsync(tmp.data(), m->d_dbg, (size_t)(span * K * 4), hipMemcpyDeviceToHost, m->stream));
        HIPTRY(m, hipStreamSynchronize(m->stream));
        for (int64_t i = 0; i < n; ++i)
            std::memcpy(out + (r + i) * K, tmp.data() + i * stride * K, (size_t)K * 4);
        r += n;
    }
    return LM_OK;
}

extern "C" void lm_debug_fail_alloc(int64_t n) {
    g_fail_at.store(n > 0 ? g_alloc_count.load() + (long)n : 0L);
}

extern "C" int64_t lm_debug_alloc_count(void) { return g_alloc_count.load(); }

extern "C" lm_status lm_debug_gemv(lm_model* m, int32_t layer, int32_t which, int32_t n_seq, const float* x,
                                   float* y) {
    if (!m || !x || !y) return LM_E_ARG;
    if (which < 0 || which > 4) return fail(m, LM_E_ARG, "lm_debug_gemv: which = %d; expected 0..4", which);
    if (which < 4 && (layer < 0 || layer >= m->cfg.n_layers))
        return fail(m, LM_E_ARG, "lm_debug_gemv: layer = %d; expected 0..%d", layer, m->cfg.n_layers - 1);
    if (n_seq < 1 || n_seq > m->cfg.max_seqs)
        return fail(m, LM_E_ARG, "lm_debug_gemv: n_seq = %d; expected 1..%d (max_seqs)", n_seq, m->cfg.max_seqs);
    if (which < 4 && layer_streamed(m, layer))
        return fail(m, LM_E_STATE, "lm_debug_gemv: layer %d is streamed (make it resident first)", layer);
    const int mats[4] = {M_QKV, M_WO, M_GU, M_DOWN};
    const QMat w = which == 4 ? lm_head_mat(m) : mat_at(m, m->d_layers + (int64_t)layer * m->blob_bytes, mats[which]);
    const int64_t K = w.K, N = w.N;
    HIPTRY(m, hipStreamSynchronize(m->stream));
    float* d = nullptr;
    HIPTRY(m, hipMalloc(&d, (size_t)(n_seq * (K + N)) * 4));
    GemvArgs a{};
    a.w = w;
    a.qtype = m->cfg.qtype;
    a.xin = d;
    a.x_stride = (int)K;
    a.out = d + n_seq * K;
    a.out_stride = (int)N;
    a.n_seq = n_seq;
    hipError_t e = hipMemcpyAsync(d, x, (size_t)(n_seq * K) * 4, hipMemcpyHostToDevice, m->stream);
    if (e == hipSuccess) e = hipMemsetAsync(d + n_seq * K, 0, (size_t)(n_seq * N) * 4, m->stream);
    if (e == hipSuccess) e = gemv(m, a, EPI_RESID, n_seq, m->stream);
    if (e == hipSuccess) e = hipMemcpyAsync(y, d + n_seq * K, (size_t)(n_seq * N) * 4, hipMemcpyDeviceToHost, m->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(m->stream);
    (void)hipFree(d);
    if (e != hipSuccess) return fail(m, LM_E_HIP, "lm_debug_gemv: %s", hipGetErrorString(e));
    return LM_OK;
}

extern "C" lm_status lm_debug_read_bw(lm_model* m, int64_t n_bytes, int32_t iters, double* ms) {
    if (!m || !ms || iters < 1) return LM_E_ARG;
    const uint8_t* buf = m->d_layers;
    const int64_t avail = (int64_t)m->n_res * m->blob_bytes;
    if (!buf || n_bytes < 16 || n_bytes > avail || n_bytes % 16)
        return fail(m, LM_E_ARG, "lm_debug_read_bw: n_bytes = %lld; expected a multiple of 16 in 16..%lld "
                    "(resident weight arena)", (long long)n_bytes, (long long)avail);
    hipEvent_t a = nullptr, b = nullptr;
    HIPTRY(m, hipEventCreate(&a));
    HIPTRY(m, hipEventCreate(&b));
    hipError_t e = launch_read_bw(buf, n_bytes, m->d_sink, m->stream);  // warm-up
    if (e == hipSuccess) e = hipEventRecord(a, m->stream);
    for (int i = 0; i < iters && e == hipSuccess; ++i) e = launch_read_bw(buf, n_bytes, m->d_sink, m->stream);
    if (e == hipSuccess) e = hipEventRecord(b, m->stream);
    if (e == hipSuccess) e = hipEventSynchronize(b);
    float t = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, a, b);
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    if (e != hipSuccess) return fail(m, LM_E_HIP, "lm_debug_read_bw: %s", hipGetErrorString(e));
    *ms = (double)t / iters;
    return LM_OK;
}
