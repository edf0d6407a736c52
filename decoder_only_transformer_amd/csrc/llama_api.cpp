// Host side of the C ABI declared in include/llama_mi355x.h: argument validation, workspace
// carve-up, RoPE table, and the per-call launch plan of Transformer.forward.
//
// Launch plan ("Llama 2 Reference Implementation -- Administrator & Developer Guide",
// section 8.4: embed -> n_layers pre-norm blocks -> final norm -> output projection):
//   prefill, bf16 and fp16: embed | per layer: rmsnorm->16-bit, MFMA [wq;wk;wv] (+RoPE, KV
//                   append), attention, MFMA wo (+residual), rmsnorm->16-bit, MFMA [w1;w3]
//                   (+SiLU gate), MFMA w2 (+residual) | final norm fused into the vocab projection.
//   decode at batch <= 4 (and the fp32 path): embed | per layer: GEMV [wq;wk;wv] with fused
//                   RMSNorm, split attention (+merge), GEMV wo (+residual), GEMV [w1;w3] with
//                   fused RMSNorm (+SiLU gate), GEMV w2 (+residual) | fused final norm + vocab GEMV.
//   decode at batch 5..32 (16-bit): the same blocks with the products on the skinny MFMA
//                   kernel; above 32 rows, the prefill GEMMs with the decode attention.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <cstdlib>
#include <map>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "../../include/llama_mi355x.h"
#include "kernels.h"

using namespace llk;

// Scratch of the allocation-free decode step (llama_decode_step_noalloc): one array per GPU,
// held until the process ends.  In host code this name is not a device address; the address
// comes from hipGetSymbolAddress, taken once per device in llama_init (g_noalloc below).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_noalloc_mu;
void* g_noalloc[kMaxDevices];   // device address of `scratch` on each device, once taken

constexpr int kMaxSplit = 32;
constexpr int kMaxSplitK = 8;      // K splits of a residual GEMM at small prefill sizes
constexpr int kSplitKRows = 512;   // prefill rows up to which split-K is considered
constexpr size_t kSplitKRowsCap = 2048;  // splits x rows the split-K workspace holds
constexpr int kSkinnyRows = 4;      // 16-bit decode batches above this use the skinny MFMA kernel
constexpr int kSkinnyMaxRows = 32;  // ... up to this many rows; larger ones the prefill GEMMs
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t k_cache, v_cache, rope, h32, q32, o32, g32, act16, g16, part, splitk, step, err, total;
    size_t splitk_floats;
    size_t kv_layer_elems;   // elements of one layer's K (or V) cache
};

int head_dim_of(const llama_args& a) { return a.dim / a.n_heads; }

// Device addresses of the per-call scratch of a forward call (everything but the KV cache and
// the RoPE table): carved from the ctx's workspace, or, for the allocation-free decode step,
// from the library's static device array.
struct Bufs {
    float *h32, *q32, *o32, *g32, *part, *splitk;
    void *act16, *g16;
    StepState* step;
    size_t splitk_floats;
};

llama_status check_args(const llama_args* a) {
    if (!a) return LLAMA_ERR_INVALID_ARG;
    if (a->dim <= 0 || a->n_layers <= 0 || a->n_heads <= 0 || a->n_kv_heads <= 0 ||
        a->vocab_size <= 0 || a->hidden_dim <= 0 || a->max_batch_size <= 0 ||
        a->max_seq_len <= 0)
        return LLAMA_ERR_INVALID_ARG;
    if (!(a->norm_eps >= 0.f) || !(a->rope_theta > 0.f)) return LLAMA_ERR_INVALID_ARG;
    if (a->dtype != LLAMA_BF16 && a->dtype != LLAMA_FP32 && a->dtype != LLAMA_FP16) return LLAMA_ERR_INVALID_ARG;
    if (a->dim % a->n_heads != 0) return LLAMA_ERR_INVALID_ARG;
    if (a->n_heads % a->n_kv_heads != 0) return LLAMA_ERR_INVALID_ARG;
    const int hd = head_dim_of(*a);
    if (hd != 32 && hd != 64 && hd != 128) return LLAMA_ERR_UNSUPPORTED;
    const int n_rep = a->n_heads / a->n_kv_heads;
    if (n_rep != 1 && n_rep != 2 && n_rep != 4 && n_rep != 8) return LLAMA_ERR_UNSUPPORTED;
    if (a->dim % 64 != 0 || a->hidden_dim % 64 != 0 || (a->n_heads * hd) % 64 != 0)
        return LLAMA_ERR_UNSUPPORTED;
    if (a->vocab_size % 2 != 0) return LLAMA_ERR_UNSUPPORTED;
    if (a->max_seq_len > 65536) return LLAMA_ERR_UNSUPPORTED;
    return LLAMA_OK;
}

// Widest B-row space of a prefill GEMM on the LDS-ring kernel (256-column tiles; the [w1;w3]
// product interleaves both matrices, so 2 * hidden_dim).
size_t splitk_cols(const llama_args& a) {
    const size_t hd = head_dim_of(a);
    const size_t widest = std::max({(size_t)a.n_heads * hd + 2 * (size_t)a.n_kv_heads * hd,
                                    2 * (size_t)a.hidden_dim, (size_t)a.dim});
    return (widest + 255) / 256 * 256;
}

Layout layout_of(const llama_args& a) {
    Layout L{};
    const size_t esz = a.dtype == LLAMA_FP32 ? 4 : 2;
    const size_t hd = head_dim_of(a);
    const size_t nq = (size_t)a.n_heads * hd;
    const size_t maxB = a.max_batch_size, maxS = a.max_seq_len;
    const size_t maxT = maxB * maxS;
    // fp32 models run everything on the vector path, which keeps every row's activations in
    // fp32 and needs none of the MFMA path's 16-bit operands or split-K partials; bf16 and
    // fp16 models prefill on MFMA and keep fp32 activations for decode rows only
    const bool fp32 = a.dtype == LLAMA_FP32;
    const size_t rows32 = fp32 ? maxT : maxB;
    L.kv_layer_elems = maxB * maxS * (size_t)a.n_kv_heads * hd;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    L.k_cache = take(L.kv_layer_elems * a.n_layers * esz);
    L.v_cache = take(L.kv_layer_elems * a.n_layers * esz);
    L.rope = take(maxS * (hd / 2) * sizeof(float) * 2);
    L.h32 = take(maxT * a.dim * sizeof(float));
    L.q32 = take(maxT * nq * sizeof(float));
    L.o32 = take(rows32 * nq * sizeof(float));
    L.g32 = take(rows32 * (size_t)a.hidden_dim * sizeof(float));
    // 16-bit activations: row-major prefill rows, or fragment-major decode rows (up to 32,
    // padding included)
    const size_t rows16 = std::max(maxT, (size_t)32);
    L.act16 = fp32 ? off : take(rows16 * (size_t)(a.dim > (int)nq ? a.dim : (int)nq) * 2);
    L.g16 = fp32 ? off : take(rows16 * (size_t)a.hidden_dim * 2);
    L.part = take(maxB * (size_t)a.n_heads * kMaxSplit * (hd + 2) * sizeof(float));
    // split-K partials of the residual GEMMs, used while a prefill has at most kSplitKRows rows
    // split-K partials: small-tile residual GEMMs (kMaxSplitK x 512 rows x dim) and short
    // prefills on the LDS-ring kernel (splits x rows x B rows, capped at kSplitKRowsCap rows)
    L.splitk_floats = fp32 ? 0 : std::max((size_t)kMaxSplitK * std::min(maxT, (size_t)kSplitKRows) * a.dim,
                                          kSplitKRowsCap * splitk_cols(a));
    L.splitk = fp32 ? off : take(L.splitk_floats * sizeof(float));
    L.step = take(sizeof(StepState));
    L.err = take(sizeof(int32_t));      // checked mode: out-of-range token flag
    L.total = off;
    return L;
}

}  // namespace

struct llama_ctx {
    llama_args a;
    llama_weights w;
    std::vector<llama_layer_weights> layers;
    Layout L;
    char* ws;
    int hd, nq, nk;
    bool bf16;      // bf16 model: the GQA decode attention on MFMA
    bool mfma16;    // bf16 or fp16 model: prefill and the skinny decode products on 16-bit MFMA
    int wtype;      // storage type of weights and KV cache (kStoreF32 / kStoreBf16 / kStoreF16)

    // decode graphs: one per (bsz, key splits), captured on a private stream
    hipStream_t cap_stream = nullptr;
    std::map<std::pair<int, int>, hipGraphExec_t> graphs;
    bool use_graphs = false;
    // checked mode (LLAMA_MI355X_CHECK_TOKENS=1 at llama_init): the embedding gather flags
    // token ids outside [0, vocab) in err, and the call returns INVALID_ARG after a sync
    bool check_tokens = false;
    int32_t* err = nullptr;

    // diagnostics: per-kernel begin/end events of the launches of one kernel class
    struct Timer : llk::KernelTimer {
        std::vector<hipEvent_t> ev;     // pairs (start, stop)
        size_t used = 0;
        bool failed = false;
        bool next_pair(hipEvent_t* start, hipEvent_t* stop) override {
            while (used + 2 > ev.size()) {
                hipEvent_t e;
                if (hipEventCreate(&e) != hipSuccess) {
                    failed = true;
                    return false;
                }
                ev.push_back(e);
            }
            *start = ev[used];
            *stop = ev[used + 1];
            used += 2;
            return true;
        }
    };
    int prof_class = 0;
    Timer timer;

    Bufs buf;       // scratch of the call in progress (see Bufs)
    void* noalloc_scratch = nullptr;   // this device's static scratch array (allocation-free decode)

    template <typename T> T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }
    size_t esz() const { return wtype == kStoreF32 ? 4 : 2; }
    void* kcache(int l) const { return ws + L.k_cache + (size_t)l * L.kv_layer_elems * esz(); }
    void* vcache(int l) const { return ws + L.v_cache + (size_t)l * L.kv_layer_elems * esz(); }
};

#define HIP_TRY(expr)                                   \
    do {                                                \
        if ((expr) != hipSuccess) return LLAMA_ERR_HIP; \
    } while (0)

namespace llk {
thread_local KernelTimer* t_kernel_timer = nullptr;
}

namespace {

// Installs the context's kernel timer on this thread for the launches of class kc, if that
// class is the one being profiled; removes it again at the end of the scope.
struct TimerScope {
    TimerScope(const llama_ctx* c, int kc) {
        if (kc != 0 && c->prof_class == kc) {
            llk::t_kernel_timer = &const_cast<llama_ctx*>(c)->timer;
            on = true;
        }
    }
    ~TimerScope() {
        if (on) llk::t_kernel_timer = nullptr;
    }
    bool on = false;
};

}  // namespace

// Launch `expr` (a hipError_t expression); its kernels are timed if class kc is profiled.
#define LAUNCH(c, kc, s, expr)                                 \
    do {                                                       \
        hipError_t e_;                                         \
        {                                                      \
            TimerScope ts_((c), (kc));                         \
            e_ = (expr);                                       \
        }                                                      \
        if (e_ != hipSuccess) return LLAMA_ERR_HIP;            \
    } while (0)

namespace {

QkvTarget qkv_target(const llama_ctx* c, int l, int start_pos, int seqlen, const StepState* st = nullptr) {
    QkvTarget t{};
    t.st = st;
    t.q = c->buf.q32;
    t.cache_k = c->kcache(l);
    t.cache_v = c->vcache(l);
    t.rope = c->at<const float2>(c->L.rope);
    t.nq = c->nq;
    t.nk = c->nk;
    t.head_dim = c->hd;
    t.max_seq = c->a.max_seq_len;
    t.start_pos = start_pos;
    t.seqlen = seqlen;
    return t;
}

// Attention over `rows` query rows (row t = batch t / seqlen, position start_pos + t % seqlen).
// Key splits of a decode step of `rows` rows at context ctx.
int decode_splits(const llama_ctx* c, int rows, int ctx) {
    const int n_rep = c->a.n_heads / c->a.n_kv_heads;
    // keys one workgroup takes in one round: 16-lane slots x 4 keys (vector kernel), or two
    // 64-key tiles (MFMA kernel for bf16 GQA with n_rep >= 4)
    const bool mfma = c->bf16 && n_rep >= 4;
    const int slots = mfma ? 32 : 4 * (n_rep <= 2 ? 16 : 8);
    const int pairs = rows * c->a.n_kv_heads;
    // workgroups wanted: about one per CU for the MFMA kernel (more splits cost more in
    // per-workgroup start-up than they gain), two per CU for the vector kernel
    const int want = ((mfma ? 256 : 512) + pairs - 1) / pairs;
    const int by_len = (ctx + 4 * slots - 1) / (4 * slots);
    return std::max(1, std::min(kMaxSplit, std::min(want, by_len)));
}

llama_status run_attention(const llama_ctx* c, int l, int rows, int seqlen, int start_pos,
                           void* out, bool out_bf16, bool allow_split, hipStream_t s,
                           const StepState* st = nullptr, int graph_splits = 0, int out_frag_mt = 0) {
    AttnArgs at{};
    at.q = c->buf.q32;
    at.cache_k = c->kcache(l);
    at.cache_v = c->vcache(l);
    at.out = out;
    at.out_bf16 = out_bf16 ? 1 : 0;
    at.out_frag_mt = out_frag_mt;
    at.part = c->buf.part;
    at.rows = rows;
    at.n_heads = c->a.n_heads;
    at.n_kv_heads = c->a.n_kv_heads;
    at.head_dim = c->hd;
    at.max_seq = c->a.max_seq_len;
    at.start_pos = start_pos;
    at.seqlen = seqlen;
    at.scale = 1.0f / std::sqrt((float)c->hd);
    at.st = st;
    if (st) {
        // graph replay: split count fixed at capture, keys per split derived in the kernel
        at.n_split = graph_splits;
        at.chunk = 0;
    } else {
        // split the keys only when there are too few (row, kv head) pairs to fill the chip,
        // and never below one round of loads per workgroup (slots x 4 keys)
        const int ctx = start_pos + seqlen;   // longest visible prefix among the rows
        int n_split = allow_split ? decode_splits(c, rows, ctx) : 1;
        int chunk = (ctx + n_split - 1) / n_split;
        chunk = (chunk + 15) / 16 * 16;
        n_split = (ctx + chunk - 1) / chunk;
        at.n_split = n_split;
        at.chunk = chunk;
    }
    LAUNCH(c, seqlen == 1 ? LLAMA_KC_ATTN_DECODE : LLAMA_KC_ATTN_PREFILL, s, launch_attn_rows(c->wtype, at, s));
    return LLAMA_OK;
}

// One transformer block on the GEMV (VALU) path for M activation rows.
llama_status block_gemv(const llama_ctx* c, int l, int M, int seqlen, int start_pos,
                        bool allow_split, hipStream_t s, const StepState* st = nullptr,
                        int graph_splits = 0) {
    const llama_layer_weights& W = c->layers[l];
    const int D = c->a.dim, F = c->a.hidden_dim;
    float* h = c->buf.h32;
    float* o32 = c->buf.o32;
    float* g32 = c->buf.g32;
    const int wb = c->wtype;

    GemvArgs g{};
    g.x = h; g.ldx = D; g.M = M; g.K = D; g.N = c->nq + 2 * c->nk;
    g.norm_w = W.attention_norm; g.eps = c->a.norm_eps;
    g.w0 = W.wq; g.w1 = W.wk; g.w2 = W.wv;
    g.qkv = qkv_target(c, l, start_pos, seqlen, st);
    LAUNCH(c, LLAMA_KC_GEMV_QKV, s, launch_gemv(wb, EPI_QKV, g, s));

    const llama_status ast = run_attention(c, l, M, seqlen, start_pos, o32, false, allow_split, s,
                                           st, graph_splits);
    if (ast != LLAMA_OK) return ast;

    g = GemvArgs{};
    g.x = o32; g.ldx = c->nq; g.M = M; g.K = c->nq; g.N = D;
    g.w0 = W.wo; g.resid = h; g.ldr = D;
    LAUNCH(c, LLAMA_KC_GEMV_WO, s, launch_gemv(wb, EPI_RESID, g, s));

    g = GemvArgs{};
    g.x = h; g.ldx = D; g.M = M; g.K = D; g.N = F;
    g.norm_w = W.ffn_norm; g.eps = c->a.norm_eps;
    g.w0 = W.w1; g.w1 = W.w3; g.out = g32; g.ldo = F;
    LAUNCH(c, LLAMA_KC_GEMV_W13, s, launch_gemv(wb, EPI_SWIGLU, g, s));

    g = GemvArgs{};
    g.x = g32; g.ldx = F; g.M = M; g.K = F; g.N = D;
    g.w0 = W.w2; g.resid = h; g.ldr = D;
    LAUNCH(c, LLAMA_KC_GEMV_W2, s, launch_gemv(wb, EPI_RESID, g, s));
    return LLAMA_OK;
}

// K splits for a residual GEMM of T rows and N = dim columns: enough workgroups to cover the
// chip (~2 per CU) while keeping at least 8 BK-steps per split.
int residual_splits(const llama_ctx* c, int T, int K) {
    if (T > kSplitKRows) return 1;
    const int bm = T <= 64 ? 64 : 128, bn = 64;
    const int tiles = ((T + bm - 1) / bm) * ((c->a.dim + bn - 1) / bn);
    int sp = (512 + tiles - 1) / tiles;
    sp = std::min(sp, std::max(1, K / 64 / 8));
    return std::max(1, std::min(sp, kMaxSplitK));
}

// K splits of the skinny wo and w2 products at M rows; their partials [splits][M][dim] sit in
// the split-K region (idle during a decode step; it holds 8 x min(rows, 512) x dim floats or
// more, and M <= 32 rows of the batch) until the RMSNorm that follows adds them to h.
int wo_splits(const llama_ctx* c, int M) { return skinny_resid_splits(M, c->a.dim, c->nq); }
int w2_splits(const llama_ctx* c, int M) { return skinny_resid_splits(M, c->a.dim, c->a.hidden_dim); }

// Scratch of one decode step of bsz <= kSkinnyMaxRows rows whose longest row attends over ctx
// keys, carved from `base` in the order of layout_of: the residual rows, q, the vector path's
// fp32 operands, the MFMA path's 16-bit operands (fragment-major, 32 rows with padding), the
// attention split partials at the split count this step takes, and the skinny residual
// products' K-split partials.  Returns the bytes needed; fills *out when base is not null.
size_t decode_scratch(const llama_ctx* c, int bsz, int ctx, char* base, Bufs* out) {
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    const size_t D = c->a.dim, F = c->a.hidden_dim, nq = c->nq, B = bsz;
    const size_t h32 = take(B * D * 4), q32 = take(B * nq * 4), o32 = take(B * nq * 4), g32 = take(B * F * 4);
    const size_t rows16 = kSkinnyMaxRows;
    const size_t act16 = c->mfma16 ? take(rows16 * std::max(D, nq) * 2) : off;
    const size_t g16 = c->mfma16 ? take(rows16 * F * 2) : off;
    const size_t part = take(B * (size_t)c->a.n_heads * decode_splits(c, bsz, ctx) * (c->hd + 2) * 4);
    const bool skinny = c->mfma16 && bsz > kSkinnyRows;
    const size_t splitk_floats = skinny ? (size_t)std::max(wo_splits(c, bsz), w2_splits(c, bsz)) * B * D : 0;
    const size_t splitk = take(splitk_floats * 4);
    if (base && out) {
        *out = Bufs{reinterpret_cast<float*>(base + h32), reinterpret_cast<float*>(base + q32),
                    reinterpret_cast<float*>(base + o32), reinterpret_cast<float*>(base + g32),
                    reinterpret_cast<float*>(base + part), reinterpret_cast<float*>(base + splitk),
                    base + act16, base + g16, nullptr, splitk_floats};
    }
    return off;
}

// One decode block for a 16-bit model at batch > kSkinnyRows: projections on the skinny MFMA
// kernel, whose activation operands (RMSNorm output, attention output, SiLU gate) are written
// in the storage type, in fragment-major order for MT = ceil(M / 16) row tiles.  The attention norm takes in
// the previous block's w2 partials, the FFN norm this block's wo partials.
llama_status block_skinny(const llama_ctx* c, int l, int M, int start_pos, hipStream_t s,
                          const StepState* st, int graph_splits) {
    const llama_layer_weights& W = c->layers[l];
    const int D = c->a.dim, F = c->a.hidden_dim;
    const int mt = (M + 15) / 16;
    float* h = c->buf.h32;
    void* act = c->buf.act16;
    void* g16 = c->buf.g16;
    float* part = c->buf.splitk;
    const int s_wo = wo_splits(c, M), s_w2 = w2_splits(c, M);
    if ((size_t)std::max(s_wo, s_w2) * M * D > c->buf.splitk_floats) return LLAMA_ERR_WORKSPACE;

    LAUNCH(c, LLAMA_KC_RMSNORM, s, launch_rmsnorm_bf16(h, D, M, D, W.attention_norm, c->a.norm_eps, act, 0, mt, s,
                                                       part, l > 0 ? s_w2 : 0, c->wtype));
    SkinnyArgs k{};
    k.wtype = c->wtype;
    k.x = act; k.M = M; k.K = D; k.N = c->nq + 2 * c->nk;
    k.w0 = W.wq; k.w1 = W.wk; k.w2 = W.wv;
    k.qkv = qkv_target(c, l, start_pos, 1, st);
    LAUNCH(c, LLAMA_KC_GEMV_QKV, s, launch_skinny(EPI_QKV, k, s));

    const llama_status ast = run_attention(c, l, M, 1, start_pos, act, true, true, s, st, graph_splits, mt);
    if (ast != LLAMA_OK) return ast;

    k = SkinnyArgs{};
    k.wtype = c->wtype;
    k.x = act; k.M = M; k.K = c->nq; k.N = D;
    k.w0 = W.wo; k.resid = h; k.ldr = D; k.ksplit = s_wo; k.part = part;
    LAUNCH(c, LLAMA_KC_GEMV_WO, s, launch_skinny(EPI_RESID, k, s));

    LAUNCH(c, LLAMA_KC_RMSNORM, s, launch_rmsnorm_bf16(h, D, M, D, W.ffn_norm, c->a.norm_eps, act, 0, mt, s,
                                                       part, s_wo, c->wtype));
    k = SkinnyArgs{};
    k.wtype = c->wtype;
    k.x = act; k.M = M; k.K = D; k.N = F;
    k.w0 = W.w1; k.w1 = W.w3; k.out16 = g16; k.out_frag_mt = mt;
    LAUNCH(c, LLAMA_KC_GEMV_W13, s, launch_skinny(EPI_SWIGLU, k, s));

    k = SkinnyArgs{};
    k.wtype = c->wtype;
    k.x = g16; k.M = M; k.K = F; k.N = D;
    k.w0 = W.w2; k.resid = h; k.ldr = D; k.ksplit = s_w2; k.part = part;
    LAUNCH(c, LLAMA_KC_GEMV_W2, s, launch_skinny(EPI_RESID, k, s));
    return LLAMA_OK;
}

// One transformer block on the 16-bit MFMA path (bf16 or fp16 model) for T = bsz*seqlen prefill
// rows (or decode rows of a large 16-bit batch).  Residual products split over K (short
// prefills) leave their partials for the RMSNorm that follows to fold into h: wo's for the FFN
// norm; w2's for the next block's attention norm.  *pending: in, the K splits of the previous
// block's w2 partials (0: none); out, this block's (0 for the last block, whose w2 adds its
// result itself: the final norm reads h directly).
llama_status block_mfma(const llama_ctx* c, int l, int T, int seqlen, int start_pos, hipStream_t s,
                        int* pending, bool decode = false) {
    const llama_layer_weights& W = c->layers[l];
    const int D = c->a.dim, F = c->a.hidden_dim;
    float* h = c->buf.h32;
    void* act = c->buf.act16;
    void* g16 = c->buf.g16;

    // deferred partials are [splits][T][dim] in the split-K region
    auto fits = [&](int parts) { return (size_t)parts * T * D <= c->buf.splitk_floats; };
    if (!fits(*pending)) return LLAMA_ERR_WORKSPACE;
    LAUNCH(c, LLAMA_KC_RMSNORM, s, launch_rmsnorm_bf16(h, D, T, D, W.attention_norm, c->a.norm_eps, act, D, 0, s,
                                                       *pending > 0 ? c->buf.splitk : nullptr, *pending, c->wtype));
    *pending = 0;
    GemmArgs g{};
    g.wtype = c->wtype;
    g.a = act; g.lda = D; g.M = T; g.K = D; g.N = c->nq + 2 * c->nk;
    g.w0 = W.wq; g.w1 = W.wk; g.w2 = W.wv;
    g.qkv = qkv_target(c, l, start_pos, seqlen);
    g.part = c->buf.splitk; g.part_cap = c->buf.splitk_floats;
    LAUNCH(c, LLAMA_KC_GEMM_QKV, s, launch_gemm(EPI_QKV, g, s));

    if (decode) {
        // single-token rows: the decode attention kernel (key splits allowed)
        llama_status st = run_attention(c, l, T, 1, start_pos, act, true, true, s);
        if (st != LLAMA_OK) return st;
    } else if (c->hd == 64 || c->hd == 128) {
        FlashArgs fa{};
        fa.q = c->buf.q32;
        fa.cache_k = c->kcache(l);
        fa.cache_v = c->vcache(l);
        fa.out = act;
        fa.bsz = T / seqlen;
        fa.seqlen = seqlen;
        fa.start_pos = start_pos;
        fa.n_heads = c->a.n_heads;
        fa.n_kv_heads = c->a.n_kv_heads;
        fa.head_dim = c->hd;
        fa.max_seq = c->a.max_seq_len;
        fa.scale = 1.0f / std::sqrt((float)c->hd);
        fa.wtype = c->wtype;
        LAUNCH(c, LLAMA_KC_ATTN_PREFILL, s, launch_flash_prefill(fa, s));
    } else {
        llama_status st = run_attention(c, l, T, seqlen, start_pos, act, true, false, s);
        if (st != LLAMA_OK) return st;
    }

    g = GemmArgs{};
    g.wtype = c->wtype;
    g.a = act; g.lda = c->nq; g.M = T; g.K = c->nq; g.N = D;
    g.w0 = W.wo; g.resid = h; g.ldr = D;
    g.splits = residual_splits(c, T, c->nq); g.part = c->buf.splitk; g.part_cap = c->buf.splitk_floats;
    int wo_parts = 0;
    g.deferred = &wo_parts;
    LAUNCH(c, LLAMA_KC_GEMM_WO, s, launch_gemm(EPI_RESID, g, s));

    if (!fits(wo_parts)) return LLAMA_ERR_WORKSPACE;
    LAUNCH(c, LLAMA_KC_RMSNORM, s, launch_rmsnorm_bf16(h, D, T, D, W.ffn_norm, c->a.norm_eps, act, D, 0, s,
                                                       wo_parts > 0 ? c->buf.splitk : nullptr, wo_parts, c->wtype));
    g = GemmArgs{};
    g.wtype = c->wtype;
    g.a = act; g.lda = D; g.M = T; g.K = D; g.N = F;
    g.w0 = W.w1; g.w1 = W.w3; g.out16 = g16; g.ldo16 = F;
    g.part = c->buf.splitk; g.part_cap = c->buf.splitk_floats;
    LAUNCH(c, LLAMA_KC_GEMM_W13, s, launch_gemm(EPI_SWIGLU, g, s));

    g = GemmArgs{};
    g.wtype = c->wtype;
    g.a = g16; g.lda = F; g.M = T; g.K = F; g.N = D;
    g.w0 = W.w2; g.resid = h; g.ldr = D;
    g.splits = residual_splits(c, T, F); g.part = c->buf.splitk; g.part_cap = c->buf.splitk_floats;
    if (l + 1 < c->a.n_layers) g.deferred = pending;
    LAUNCH(c, LLAMA_KC_GEMM_W2, s, launch_gemm(EPI_RESID, g, s));
    return LLAMA_OK;
}

// Final RMSNorm + output projection for `rows` rows of h spaced `ldx` floats apart.
llama_status final_logits(const llama_ctx* c, const float* x, int64_t ldx, int rows, float* logits,
                          hipStream_t s, const StepState* st = nullptr) {
    GemvArgs g{};
    g.st = st;
    g.x = x; g.ldx = ldx; g.M = rows; g.K = c->a.dim; g.N = c->a.vocab_size;
    g.norm_w = c->w.norm; g.eps = c->a.norm_eps;
    g.w0 = c->w.output; g.out = logits; g.ldo = c->a.vocab_size;
    LAUNCH(c, LLAMA_KC_GEMV_OUT, s, launch_gemv(c->wtype, EPI_STORE, g, s));
    return LLAMA_OK;
}

// Checked mode: the flag the embedding gather set during the call, read after the stream has
// drained; INVALID_ARG if a token id was outside [0, vocab).
llama_status finish_token_check(const llama_ctx* c, llama_status r, hipStream_t s) {
    if (!c->check_tokens || r != LLAMA_OK) return r;
    int32_t flag = 0;
    if (hipMemcpyAsync(&flag, c->err, sizeof flag, hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return LLAMA_ERR_HIP;
    return flag ? LLAMA_ERR_INVALID_ARG : LLAMA_OK;
}

}  // namespace

extern "C" {

llama_status llama_check_args(const llama_args* a) { return check_args(a); }

size_t llama_workspace_bytes(const llama_args* a) {
    if (check_args(a) != LLAMA_OK) return 0;
    return layout_of(*a).total;
}

llama_status llama_init(const llama_args* a, const llama_weights* w, void* d_workspace,
                        size_t workspace_bytes, void* stream, llama_ctx** out) {
    if (out) *out = nullptr;
    if (!out || !w) return LLAMA_ERR_INVALID_ARG;
    const llama_status st = check_args(a);
    if (st != LLAMA_OK) return st;
    if (!w->tok_embeddings || !w->norm || !w->output || !w->layers) return LLAMA_ERR_INVALID_ARG;
    for (const void* q : {w->tok_embeddings, w->norm, w->output})
        if (reinterpret_cast<uintptr_t>(q) & 15) return LLAMA_ERR_INVALID_ARG;
    for (int l = 0; l < a->n_layers; ++l) {
        const llama_layer_weights& L = w->layers[l];
        const void* p[9] = {L.attention_norm, L.wq, L.wk, L.wv, L.wo, L.ffn_norm, L.w1, L.w2, L.w3};
        for (const void* q : p)
            if (!q || (reinterpret_cast<uintptr_t>(q) & 15)) return LLAMA_ERR_INVALID_ARG;
    }
    const Layout L = layout_of(*a);
    if (!d_workspace || workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(d_workspace) % kAlign))
        return LLAMA_ERR_WORKSPACE;

    llama_ctx* c = new (std::nothrow) llama_ctx();
    if (!c) return LLAMA_ERR_INVALID_ARG;
    c->a = *a;
    c->w = *w;
    c->layers.assign(w->layers, w->layers + a->n_layers);
    c->w.layers = c->layers.data();
    c->L = L;
    c->ws = static_cast<char*>(d_workspace);
    c->hd = head_dim_of(*a);
    c->nq = a->n_heads * c->hd;
    c->nk = a->n_kv_heads * c->hd;
    c->bf16 = a->dtype == LLAMA_BF16;
    c->mfma16 = a->dtype != LLAMA_FP32;
    c->buf = Bufs{c->at<float>(L.h32), c->at<float>(L.q32), c->at<float>(L.o32), c->at<float>(L.g32),
                  c->at<float>(L.part), c->at<float>(L.splitk), c->at<void>(L.act16), c->at<void>(L.g16),
                  c->at<StepState>(L.step), L.splitk_floats};
    c->wtype = a->dtype == LLAMA_BF16 ? kStoreBf16 : (a->dtype == LLAMA_FP16 ? kStoreF16 : kStoreF32);
    {
        // Graph replay of decode steps is opt-in: measured on this stack, replaying the
        // captured step is no faster than launching its kernels back to back.
        const char* g = std::getenv("LLAMA_MI355X_GRAPHS");
        c->use_graphs = g && g[0] == '1';
        const char* ck = std::getenv("LLAMA_MI355X_CHECK_TOKENS");
        c->check_tokens = ck && ck[0] == '1';
        c->err = c->at<int32_t>(L.err);
    }

    // RoPE table: entry (t, i) = (cos, sin) of t * theta^(-2i/hd), computed in float64.
    const int half = c->hd / 2;
    std::vector<float> tab((size_t)a->max_seq_len * half * 2);
    for (int t = 0; t < a->max_seq_len; ++t)
        for (int i = 0; i < half; ++i) {
            const double f = std::pow((double)a->rope_theta, -2.0 * i / c->hd);
            const double ang = (double)t * f;
            tab[((size_t)t * half + i) * 2] = (float)std::cos(ang);
            tab[((size_t)t * half + i) * 2 + 1] = (float)std::sin(ang);
        }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(c->ws + L.rope, tab.data(), tab.size() * sizeof(float), hipMemcpyHostToDevice, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess) {
        delete c;
        return LLAMA_ERR_HIP;
    }
    // this device's copy of the static scratch of the allocation-free decode step
    int dev = -1;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
        std::lock_guard<std::mutex> lock(g_noalloc_mu);
        if (!g_noalloc[dev]) {
            void* p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess)
                g_noalloc[dev] = p;
            else
                (void)hipGetLastError();   // leave no error for the next call to report
        }
        c->noalloc_scratch = g_noalloc[dev];
    }
    *out = c;
    return LLAMA_OK;
}

static llama_status prefill_plan(llama_ctx* c, const int32_t* d_tokens, int64_t ld_tokens, int32_t bsz,
                                 int32_t seqlen, int32_t start_pos, float* d_logits, int32_t all_positions,
                                 hipStream_t s);

llama_status llama_prefill(llama_ctx* c, const int32_t* d_tokens, int64_t ld_tokens, int32_t bsz,
                           int32_t seqlen, int32_t start_pos, float* d_logits,
                           int32_t all_positions, void* stream) {
    if (!c || !d_tokens || !d_logits) return LLAMA_ERR_INVALID_ARG;
    if (bsz < 1 || bsz > c->a.max_batch_size || seqlen < 1 || start_pos < 0 ||
        (int64_t)start_pos + seqlen > c->a.max_seq_len || ld_tokens < seqlen)
        return LLAMA_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (c->check_tokens) HIP_TRY(launch_clear_flag(c->err, s));
    return finish_token_check(c, prefill_plan(c, d_tokens, ld_tokens, bsz, seqlen, start_pos, d_logits,
                                              all_positions, s), s);
}

// The launch sequence of one prefill call (arguments checked by llama_prefill).
static llama_status prefill_plan(llama_ctx* c, const int32_t* d_tokens, int64_t ld_tokens, int32_t bsz,
                                 int32_t seqlen, int32_t start_pos, float* d_logits, int32_t all_positions,
                                 hipStream_t s) {
    const int D = c->a.dim;
    const int T = bsz * seqlen;
    float* h = c->buf.h32;
    HIP_TRY(launch_embed(d_tokens, ld_tokens, bsz, seqlen, c->w.tok_embeddings, c->wtype,
                         c->a.vocab_size, D, h, nullptr, s, c->check_tokens ? c->err : nullptr));
    int pending = 0;   // K splits of the last w2 partials not yet folded into h
    for (int l = 0; l < c->a.n_layers; ++l) {
        const llama_status st = c->mfma16 ? block_mfma(c, l, T, seqlen, start_pos, s, &pending)
                                          : block_gemv(c, l, T, seqlen, start_pos, false, s);
        if (st != LLAMA_OK) return st;
    }
    float* last = h + (size_t)(seqlen - 1) * D;   // the last position of every row, seqlen * D apart
    if (!all_positions && c->mfma16 && bsz > kSkinnyRows && bsz <= kSkinnyMaxRows) {
        // 5..32 rows: the norm to fragment-major 16-bit operands and the vocab product on the
        // skinny MFMA kernel, which streams the output matrix once (the vector GEMV would
        // stream it once per 4 rows)
        void* act = c->buf.act16;
        LAUNCH(c, LLAMA_KC_RMSNORM, s, launch_rmsnorm_bf16(last, (int64_t)seqlen * D, bsz, D, c->w.norm, c->a.norm_eps,
                                                           act, 0, (bsz + 15) / 16, s, nullptr, 0, c->wtype));
        SkinnyArgs k{};
        k.wtype = c->wtype;
        k.x = act; k.M = bsz; k.K = D; k.N = c->a.vocab_size;
        k.w0 = c->w.output; k.out = d_logits; k.ldo = c->a.vocab_size;
        LAUNCH(c, LLAMA_KC_GEMV_OUT, s, launch_skinny(EPI_STORE, k, s));
        return LLAMA_OK;
    }
    if (!all_positions) return final_logits(c, last, (int64_t)seqlen * D, bsz, d_logits, s);
    if (!c->mfma16) return final_logits(c, h, D, T, d_logits, s);
    void* act = c->buf.act16;
    HIP_TRY(launch_rmsnorm_bf16(h, D, T, D, c->w.norm, c->a.norm_eps, act, D, 0, s, nullptr, 0, c->wtype));
    GemmArgs g{};
    g.wtype = c->wtype;
    g.a = act; g.lda = D; g.M = T; g.K = D; g.N = c->a.vocab_size;
    g.w0 = c->w.output; g.out = d_logits; g.ldo = c->a.vocab_size;
    HIP_TRY(launch_gemm(EPI_STORE, g, s));
    return LLAMA_OK;
}

// The launch sequence of one decode step.  With st, per-step values are read from the
// device step state (graph capture); otherwise they are launch arguments.
static llama_status decode_plan(llama_ctx* c, const int32_t* d_tokens, int64_t ld_tokens, int32_t bsz,
                                int32_t start_pos, float* d_logits, hipStream_t s,
                                const StepState* st, int graph_splits) {
    const int D = c->a.dim;
    float* h = c->buf.h32;
    HIP_TRY(launch_embed(d_tokens, ld_tokens, bsz, 1, c->w.tok_embeddings, c->wtype,
                         c->a.vocab_size, D, h, st, s, c->check_tokens ? c->err : nullptr));
    if (c->mfma16 && bsz > kSkinnyMaxRows) {
        // more rows than the skinny kernels take: the prefill GEMMs with the decode attention
        // (launch arguments only, so not under graph capture)
        if (st) return LLAMA_ERR_UNSUPPORTED;
        int pending = 0;
        for (int l = 0; l < c->a.n_layers; ++l) {
            const llama_status r = block_mfma(c, l, bsz, 1, start_pos, s, &pending, true);
            if (r != LLAMA_OK) return r;
        }
        return final_logits(c, h, D, bsz, d_logits, s);
    }
    const bool skinny = c->mfma16 && bsz > kSkinnyRows;
    for (int l = 0; l < c->a.n_layers; ++l) {
        const llama_status r = skinny ? block_skinny(c, l, bsz, start_pos, s, st, graph_splits)
                                      : block_gemv(c, l, bsz, 1, start_pos, true, s, st, graph_splits);
        if (r != LLAMA_OK) return r;
    }
    if (!skinny) return final_logits(c, h, D, bsz, d_logits, s, st);
    void* act = c->buf.act16;
    // the final norm takes in the last block's w2 partials
    LAUNCH(c, LLAMA_KC_RMSNORM, s, launch_rmsnorm_bf16(h, D, bsz, D, c->w.norm, c->a.norm_eps, act, 0, (bsz + 15) / 16, s,
                                                       c->buf.splitk, w2_splits(c, bsz), c->wtype));
    SkinnyArgs k{};
    k.wtype = c->wtype;
    k.x = act; k.M = bsz; k.K = D; k.N = c->a.vocab_size;
    k.w0 = c->w.output; k.out = d_logits; k.ldo = c->a.vocab_size; k.st = st;
    LAUNCH(c, LLAMA_KC_GEMV_OUT, s, launch_skinny(EPI_STORE, k, s));
    return LLAMA_OK;
}

// Captured graph of a decode step for (bsz, key splits), instantiated on first use.
static llama_status decode_graph(llama_ctx* c, int bsz, int splits, hipGraphExec_t* out) {
    const auto key = std::make_pair(bsz, splits);
    const auto it = c->graphs.find(key);
    if (it != c->graphs.end()) {
        *out = it->second;
        return LLAMA_OK;
    }
    if (!c->cap_stream && hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking) != hipSuccess)
        return LLAMA_ERR_HIP;
    const StepState* st = c->buf.step;
    if (hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal) != hipSuccess)
        return LLAMA_ERR_HIP;
    const llama_status r = decode_plan(c, nullptr, 0, bsz, 0, nullptr, c->cap_stream, st, splits);
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(c->cap_stream, &graph);
    if (r != LLAMA_OK || e != hipSuccess) {
        if (graph) (void)hipGraphDestroy(graph);
        return r != LLAMA_OK ? r : LLAMA_ERR_HIP;
    }
    hipGraphExec_t exec = nullptr;
    const hipError_t ie = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ie != hipSuccess) return LLAMA_ERR_HIP;
    c->graphs[key] = exec;
    *out = exec;
    return LLAMA_OK;
}

llama_status llama_decode_step(llama_ctx* c, const int32_t* d_tokens, int64_t ld_tokens,
                               int32_t bsz, int32_t start_pos, float* d_logits, void* stream) {
    if (!c || !d_tokens || !d_logits) return LLAMA_ERR_INVALID_ARG;
    if (bsz < 1 || bsz > c->a.max_batch_size || start_pos < 0 || start_pos >= c->a.max_seq_len ||
        ld_tokens < 1)
        return LLAMA_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (c->check_tokens) {
        HIP_TRY(launch_clear_flag(c->err, s));
        return finish_token_check(c, decode_plan(c, d_tokens, ld_tokens, bsz, start_pos, d_logits, s, nullptr, 0), s);
    }
    if (!c->use_graphs || c->prof_class != 0 || (c->mfma16 && bsz > kSkinnyMaxRows))
        return decode_plan(c, d_tokens, ld_tokens, bsz, start_pos, d_logits, s, nullptr, 0);
    // graph replay: per-step values go to the device step state, then one graph launch
    const int splits = decode_splits(c, bsz, start_pos + 1);
    hipGraphExec_t exec;
    const llama_status r = decode_graph(c, bsz, splits, &exec);
    if (r != LLAMA_OK) return r;
    HIP_TRY(launch_set_step(c->buf.step, start_pos, ld_tokens, d_tokens, d_logits, s));
    HIP_TRY(hipGraphLaunch(exec, s));
    return LLAMA_OK;
}

llama_status llama_decode_step_noalloc(llama_ctx* c, const int32_t* d_tokens, int64_t ld_tokens,
                                       int32_t bsz, int32_t start_pos, float* d_logits, void* stream) {
    if (!c || !d_tokens || !d_logits) return LLAMA_ERR_INVALID_ARG;
    if (bsz < 1 || bsz > c->a.max_batch_size || start_pos < 0 || start_pos >= c->a.max_seq_len ||
        ld_tokens < 1)
        return LLAMA_ERR_INVALID_ARG;
    if (bsz > kSkinnyMaxRows) return LLAMA_ERR_UNSUPPORTED;
    if (!c->noalloc_scratch) return LLAMA_ERR_HIP;
    Bufs b{};
    if (decode_scratch(c, bsz, start_pos + 1, static_cast<char*>(c->noalloc_scratch), &b) > kNoAllocScratchBytes)
        return LLAMA_ERR_WORKSPACE;
    // eager launches only (a graph or a timing event would be created on first use), with the
    // step's scratch in the static array; the ctx's own scratch is untouched
    const Bufs saved = c->buf;
    const int saved_prof = c->prof_class;
    c->buf = b;
    c->prof_class = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    llama_status r = c->check_tokens && launch_clear_flag(c->err, s) != hipSuccess ? LLAMA_ERR_HIP : LLAMA_OK;
    if (r == LLAMA_OK) r = finish_token_check(c, decode_plan(c, d_tokens, ld_tokens, bsz, start_pos, d_logits, s, nullptr, 0), s);
    c->buf = saved;
    c->prof_class = saved_prof;
    return r;
}

llama_status llama_argmax(const float* d_logits, int32_t bsz, int32_t vocab, int64_t row_stride,
                          int32_t* d_out, void* stream) {
    if (!d_logits || !d_out || bsz < 1 || vocab < 1 || row_stride < vocab) return LLAMA_ERR_INVALID_ARG;
    HIP_TRY(launch_argmax(d_logits, bsz, vocab, row_stride, d_out, static_cast<hipStream_t>(stream)));
    return LLAMA_OK;
}

llama_status llama_sample_top_p(const float* d_logits, int32_t bsz, int32_t vocab, int64_t row_stride,
                                float temperature, float top_p, const float* d_uniform, int32_t* d_out,
                                float* d_logprob, void* stream) {
    if (!d_logits || !d_uniform || !d_out || bsz < 1 || vocab < 1 || row_stride < vocab ||
        !(temperature > 0.f) || !std::isfinite(temperature) || !(top_p >= 0.f))
        return LLAMA_ERR_INVALID_ARG;
    if (vocab > kMaxSampleVocab) return LLAMA_ERR_UNSUPPORTED;
    HIP_TRY(launch_sample_top_p(d_logits, bsz, vocab, row_stride, temperature, top_p, d_uniform, d_out, d_logprob,
                                static_cast<hipStream_t>(stream)));
    return LLAMA_OK;
}

llama_status llama_select_next(const int32_t* d_next, int32_t* d_tokens, int64_t ld_tokens,
                               int32_t cur_pos, const int32_t* d_prompt_len, int32_t bsz,
                               void* stream) {
    if (!d_next || !d_tokens || !d_prompt_len || bsz < 1 || cur_pos < 0 || cur_pos >= ld_tokens)
        return LLAMA_ERR_INVALID_ARG;
    HIP_TRY(launch_select(d_next, d_tokens, ld_tokens, cur_pos, d_prompt_len, bsz,
                          static_cast<hipStream_t>(stream)));
    return LLAMA_OK;
}

llama_status llama_profile_select(llama_ctx* c, int32_t kernel_class) {
    if (!c || kernel_class < 0 || kernel_class >= LLAMA_KC_COUNT) return LLAMA_ERR_INVALID_ARG;
    c->prof_class = kernel_class;
    return LLAMA_OK;
}

llama_status llama_profile_read(llama_ctx* c, int64_t* launches, double* total_ms) {
    if (!c || !launches || !total_ms) return LLAMA_ERR_INVALID_ARG;
    auto& T = c->timer;
    double ms = 0.0;
    const size_t pairs = T.used / 2;
    for (size_t i = 0; i < pairs; ++i) {
        float t = 0.f;
        if (hipEventSynchronize(T.ev[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&t, T.ev[2 * i], T.ev[2 * i + 1]) != hipSuccess)
            return LLAMA_ERR_HIP;
        ms += t;
    }
    *launches = (int64_t)pairs;
    *total_ms = ms;
    T.used = 0;
    if (T.failed) {
        T.failed = false;
        return LLAMA_ERR_HIP;
    }
    return LLAMA_OK;
}

void llama_destroy(llama_ctx* c) {
    if (!c) return;
    for (hipEvent_t e : c->timer.ev) (void)hipEventDestroy(e);
    for (auto& kv : c->graphs) (void)hipGraphExecDestroy(kv.second);
    if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
    delete c;
}

const char* llama_status_str(llama_status st) {
    switch (st) {
        case LLAMA_OK: return "LLAMA_OK";
        case LLAMA_ERR_INVALID_ARG: return "LLAMA_ERR_INVALID_ARG";
        case LLAMA_ERR_UNSUPPORTED: return "LLAMA_ERR_UNSUPPORTED";
        case LLAMA_ERR_WORKSPACE: return "LLAMA_ERR_WORKSPACE";
        case LLAMA_ERR_HIP: return "LLAMA_ERR_HIP";
        case LLAMA_STATUS_MAX_ENUM: break;
    }
    return "LLAMA_STATUS_UNKNOWN";
}

}  // extern "C"
