// Launch interface between the host library (llama_api.cpp) and the gfx950 kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llk {

// Storage type of weights and KV cache, as the launchers take it.
constexpr int kStoreF32 = 0, kStoreBf16 = 1, kStoreF16 = 2;

// Per-kernel timing for diagnostics.  While a timer is installed on the calling thread,
// every kernel goes out through hipExtLaunchKernel with an event pair of its own, which HIP
// ties to that dispatch's begin and end timestamps (so queue gaps between launches are not
// counted).  With no timer installed a launch is a plain hipLaunchKernelGGL.
struct KernelTimer {
    virtual bool next_pair(hipEvent_t* start, hipEvent_t* stop) = 0;
};
extern thread_local KernelTimer* t_kernel_timer;

template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, Args... args) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (t_kernel_timer && t_kernel_timer->next_pair(&e0, &e1))
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e0, e1, 0, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shmem, s, args...);
}

enum Epilogue : int {
    EPI_QKV = 0,     // rows of [wq; wk; wv]: RoPE on q and k, q -> q buffer, k/v -> KV cache
    EPI_RESID = 1,   // resid[m][n] += y
    EPI_SWIGLU = 2,  // out[m][n] = silu(x.w1[n]) * (x.w3[n])
    EPI_STORE = 3    // out[m][n] = y (fp32 logits)
};

// Per-call values of a decode step kept in device memory, so one captured graph serves
// every position: written by a one-thread kernel before the graph is launched.
struct StepState {
    int32_t pos;            // start_pos of the step
    int32_t pad;
    int64_t ld;             // token row stride
    const int32_t* tokens;  // token of row b at tokens[b * ld]
    float* logits;          // [bsz][vocab]
};

// Row m of a call covers token (b = m / seqlen, position start_pos + m % seqlen).
struct QkvTarget {
    float* q;              // [M][nq] fp32
    void* cache_k;         // this layer's K cache base: [max_batch][max_seq][n_kv_heads][head_dim]
    void* cache_v;
    const float2* rope;    // [max_seq][head_dim/2] (cos, sin)
    int nq, nk;            // rows of wq and of wk (= n_heads*hd, n_kv_heads*hd)
    int head_dim;
    int max_seq;
    int start_pos, seqlen;
    const StepState* st;   // if set, start_pos comes from st->pos
    int row0;              // prefill GEMM paths: rows of the launch start at this row of the
                           // bsz x seqlen rectangle (decode paths: 0)
};

// y[m][n] = sum_k x[m][k] * W[n][k]  (VALU, fp32 activations, weights streamed once per
// M-chunk).  With norm_w, x is RMS-normalised on the fly: x / sqrt(mean(x^2)+eps) * norm_w
// (correctly rounded square root and division).
struct GemvArgs {
    const float* x; int64_t ldx;
    int M, K, N;           // N = output columns (SWIGLU: hidden units)
    const void* norm_w; float eps;
    const void* w0;        // [N][K] (QKV: wq; SWIGLU: w1)
    const void* w1;        // QKV: wk; SWIGLU: w3
    const void* w2;        // QKV: wv
    float* out; int64_t ldo;
    float* resid; int64_t ldr;
    QkvTarget qkv;
    const StepState* st;   // if set, the STORE epilogue writes st->logits
};

// C[m][n] = sum_k A[m][k] * W[n][k] on 16-bit MFMA, fp32 accumulate.  A [M][lda] and W in
// the storage type wtype (kStoreBf16 or kStoreF16), as are the 16-bit outputs.
struct GemmArgs {
    const void* a; int64_t lda;
    int M, K, N;           // N = output columns (SWIGLU: hidden units)
    const void* w0; const void* w1; const void* w2;
    float* out; int64_t ldo;       // STORE (fp32)
    void* out16; int64_t ldo16;    // SWIGLU (16-bit, wtype)
    float* resid; int64_t ldr;
    QkvTarget qkv;
    int splits;            // K splits of the small-tile residual GEMM: partials [splits][M][N]
    float* part;           // split-K partials (also used by short prefills on the LDS-ring kernel)
    size_t part_cap;       // floats available at `part`
    // RESID only, host pointer: if set, a product split over K leaves its fp32 partials
    // [splits][M][N] at `part` instead of adding them to resid, and stores the split count
    // here (0 when it added its result to resid itself); the caller has the RMSNorm that
    // follows fold them in (launch_rmsnorm_bf16's part / nsplit).
    int* deferred;
    int wtype = kStoreBf16;
};

constexpr int kMaxBigSplit = 16;

// y = x W^T for M <= 32 rows on 16-bit MFMA (decode with batch > 4).  x is 16-bit (wtype) in
// fragment-major order for MT = ceil(M / 16) row tiles (frag_index).
struct SkinnyArgs {
    const void* x;
    int M, K, N;           // N = output rows (SWIGLU: hidden units)
    const void* w0; const void* w1; const void* w2;
    float* out; void* out16; int64_t ldo;   // STORE (fp32) / SWIGLU (16-bit, wtype)
    int out_frag_mt;       // SWIGLU: > 0 writes out16 fragment-major for that many row tiles
    float* resid; int64_t ldr;
    int ksplit;            // RESID: > 1 splits K over gridDim.y, each split writing its sum
    float* part;           //   to part[split][M][N] in place of adding it to resid
    QkvTarget qkv;
    const StepState* st;   // if set, the STORE epilogue writes st->logits
    int wtype = kStoreBf16;    // storage type of the weights and 16-bit activations
};

// Causal attention for a set of query rows against the KV cache (one query position per
// row, all n_rep heads of one kv head per workgroup, keys split over gridDim.x).
struct AttnArgs {
    const float* q;        // [rows][n_heads*hd] fp32 (RoPE applied)
    const void* cache_k;   // layer base
    const void* cache_v;
    void* out;             // [rows][n_heads*hd], fp32, or 16-bit (out_bf16: the cache's storage
    int out_bf16;          //   type, bf16 or fp16)
    int out_frag_mt;       // 16-bit out: > 0 writes it fragment-major for that many row tiles
    float* part;           // [rows][n_heads][n_split][hd + 2] partials when n_split > 1
    int rows, n_heads, n_kv_heads, head_dim, max_seq;
    int row0;              // first row of this launch (launches are split at 65535 rows)
    int start_pos, seqlen; // row t -> b = t / seqlen, position start_pos + t % seqlen
    int n_split, chunk;    // keys per split (multiple of 16); chunk 0: derived from st
    float scale;           // 1/sqrt(head_dim)
    const StepState* st;   // if set, start_pos comes from st->pos
};

// Causal GQA attention of a prefill (16-bit MFMA): rows b*seqlen + s at positions start_pos + s.
struct FlashArgs {
    const float* q;        // [bsz*seqlen][n_heads*hd] (fp32 holding values of the storage type)
    const void* cache_k;   // layer base, storage type
    const void* cache_v;
    void* out;             // [bsz*seqlen][n_heads*hd] storage type
    int bsz, seqlen, start_pos;
    int n_heads, n_kv_heads, head_dim, max_seq;
    float scale;
    int wtype = kStoreBf16;    // kStoreBf16 or kStoreF16
};

// Temperature + top-p draw, one token per row (vocab <= kMaxSampleVocab); see sampling.hip.
constexpr int kMaxSampleVocab = 32768;
hipError_t launch_sample_top_p(const float* logits, int bsz, int vocab, int64_t stride, float temperature,
                               float top_p, const float* uniform, int32_t* out, float* logprob, hipStream_t s);
hipError_t launch_flash_prefill(const FlashArgs& a, hipStream_t s);
// RoPE, q store and K/V cache append from the sum of `splits` partial [wq; wk; wv]
// projections [splits][T][ldy] (summed in split order); row m is row t.row0 + m of the
// bsz x seqlen rectangle.
hipError_t launch_rope_scatter_parts(const float* y, int splits, int64_t ldy, int T, const QkvTarget& t,
                                     hipStream_t s, int wtype = kStoreBf16);
// err: if not null, set to 1 when a token id is outside [0, vocab) (the ids are clamped into
// range either way, so nothing outside the table is read).
hipError_t launch_embed(const int32_t* tokens, int64_t ld, int bsz, int seqlen, const void* table,
                        int wtype, int vocab, int dim, float* h, const StepState* st, hipStream_t s,
                        int32_t* err = nullptr);
// *flag = 0 (a one-thread kernel: no memset node if the stream is being captured).
hipError_t launch_clear_flag(int32_t* flag, hipStream_t s);
hipError_t launch_set_step(StepState* st, int pos, int64_t ld, const int32_t* tokens, float* logits,
                           hipStream_t s);
// RMSNorm of fp32 rows to the 16-bit storage type wtype (norm weights of that type);
// frag_mt > 0 writes the rows fragment-major (frag_index).
// nsplit > 1 (at most kMaxNormFold): h[r] += part[0][r] + ... + part[nsplit-1][r] first (the
// K-split partials [nsplit][rows][dim] of the residual product that precedes the norm),
// written back to h.
constexpr int kMaxNormFold = 16;
hipError_t launch_rmsnorm_bf16(float* h, int64_t ldh, int rows, int dim, const void* w,
                               float eps, void* out, int64_t ldo, int frag_mt, hipStream_t s,
                               const float* part = nullptr, int nsplit = 0, int wtype = kStoreBf16);
hipError_t launch_gemv(int wtype, int epi, const GemvArgs& a, hipStream_t s);   // wtype: kStore*
hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s);
hipError_t launch_skinny(int epi, const SkinnyArgs& a, hipStream_t s);
// K splits the skinny residual product of M x K by K x N takes (SkinnyArgs::ksplit).
int skinny_resid_splits(int M, int N, int K);
hipError_t launch_attn_rows(int kv_type, const AttnArgs& a, hipStream_t s);   // kv_type: kStore*
hipError_t launch_argmax(const float* logits, int bsz, int vocab, int64_t stride, int32_t* out,
                         hipStream_t s);
hipError_t launch_select(const int32_t* next, int32_t* tokens, int64_t ld, int cur_pos,
                         const int32_t* prompt_len, int bsz, hipStream_t s);

}  // namespace llk
