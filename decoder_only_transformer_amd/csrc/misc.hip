// Small bandwidth kernels: embedding gather, RMSNorm to a bf16 GEMM operand, greedy argmax,
// and the generate loop's prompt-preserving token select.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

// h[b*seqlen + s][:] = E[tokens[b*ld + s]][:] as fp32 (the residual stream is fp32).  The row
// is read as 16-byte chunks (dim is a multiple of 64 and the table 16-byte aligned), every
// load of a round issued before its stores, so a row costs one memory round trip.
template <typename WT>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tokens, int64_t ld, int seqlen,
                                                    const WT* __restrict__ table, int vocab, int dim,
                                                    float* __restrict__ h, const StepState* st,
                                                    int32_t* err) {
    if (st) {
        tokens = st->tokens;
        ld = st->ld;
    }
    const int t = blockIdx.x;
    const int b = t / seqlen, s = t - b * seqlen;
    int tok = tokens[(size_t)b * ld + s];
    if (err && (tok < 0 || tok >= vocab) && threadIdx.x == 0) *err = 1;   // checked mode
    tok = min(max(tok, 0), vocab - 1);   // out-of-range ids are a caller error; never read outside E
    constexpr int kPer = Elem<WT>::kPer16B;
    constexpr int kRound = 4;            // chunks per thread per round
    const uint4* src = reinterpret_cast<const uint4*>(table + (size_t)tok * dim);
    float* out = h + (size_t)t * dim;
    const int n = dim / kPer;
    for (int c0 = threadIdx.x; c0 < n; c0 += 256 * kRound) {
        uint4 v[kRound];
#pragma unroll
        for (int u = 0; u < kRound; ++u) {
            const int c = c0 + u * 256;
            v[u] = c < n ? src[c] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kRound; ++u) {
            const int c = c0 + u * 256;
            if (c >= n) continue;
            float f[kPer];
            Elem<WT>::unpack(v[u], f);
#pragma unroll
            for (int j = 0; j < kPer; j += 4)
                *reinterpret_cast<float4*>(out + (size_t)c * kPer + j) = make_float4(f[j], f[j + 1], f[j + 2], f[j + 3]);
        }
    }
}

// out[r][:] = bf16( h[r][:] / sqrt(mean(h[r]^2) + eps) * w ).  The squares are summed in fp64
// (each is exact there) and the mean rounded once to fp32, so it is the correctly rounded
// mean in all but ~1e-7 of rows whatever the summation order; the square root and the
// division are the correctly rounded fp32 ones (the division as div_rn with the row's
// correctly rounded reciprocal).  Where a row of bf16 values (an embedding
// row) times the scale lands on many exact bf16 ties, one bit of the denominator decides
// hundreds of roundings, so the denominator is made exact rather than approximate.
// With nsplit > 1, h[r] first takes the K-split partial sums of the residual product that
// wrote them, part[0][r] + ... + part[nsplit - 1][r] (part is [nsplit][rows][dim], summed in
// split order), and is stored back.
template <typename WT>
__global__ __launch_bounds__(256) void rmsnorm_bf16_kernel(float* h, int64_t ldh, int dim,
                                                           const WT* w, float eps, uint16_t* out,
                                                           int64_t ldo, int frag_mt,
                                                           const float* part, int nsplit) {
    __shared__ double red[4];
    float* x = h + (size_t)blockIdx.x * ldh;
    double ss = 0.0;
    for (int k = threadIdx.x * 4; k < dim; k += 256 * 4) {
        float4 v = *reinterpret_cast<const float4*>(x + k);
        if (nsplit > 1) {
            float4 p = *reinterpret_cast<const float4*>(part + (size_t)blockIdx.x * dim + k);
            for (int sp = 1; sp < nsplit; ++sp) {
                const float4 q = *reinterpret_cast<const float4*>(part + ((size_t)sp * gridDim.x + blockIdx.x) * dim + k);
                p.x += q.x; p.y += q.y; p.z += q.z; p.w += q.w;
            }
            v.x += p.x; v.y += p.y; v.z += p.z; v.w += p.w;
            *reinterpret_cast<float4*>(x + k) = v;
        }
        ss += sq64(v.x) + sq64(v.y) + sq64(v.z) + sq64(v.w);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float den = sqrtf((float)((red[0] + red[1] + red[2] + red[3]) / (double)dim) + eps);
    const float rcp = 1.0f / den;
    // row-major [rows][ldo], or fragment-major (4 consecutive k stay adjacent in both)
    for (int k = threadIdx.x * 4; k < dim; k += 256 * 4) {
        const float4 v = *reinterpret_cast<const float4*>(x + k);
        uint2 p;
        p.x = Mma<WT>::pack2(div_rn(v.x, den, rcp) * Elem<WT>::load(w, k), div_rn(v.y, den, rcp) * Elem<WT>::load(w, k + 1));
        p.y = Mma<WT>::pack2(div_rn(v.z, den, rcp) * Elem<WT>::load(w, k + 2), div_rn(v.w, den, rcp) * Elem<WT>::load(w, k + 3));
        const size_t o = frag_mt ? frag_index(blockIdx.x, k, frag_mt) : (size_t)blockIdx.x * ldo + k;
        *reinterpret_cast<uint2*>(out + o) = p;
    }
}

// Same, for rows of at most 1024 * NV elements: every load of the row (and of the weights and
// NS partials) is issued before the first use and the row stays in registers for the second
// half, so a row costs one memory round trip instead of one per chunk and pass.
template <typename T16, int NV, int NS>
__global__ __launch_bounds__(256) void rmsnorm_reg_kernel(float* h, int64_t ldh, int dim, const T16* w,
                                                          float eps, uint16_t* out, int64_t ldo, int frag_mt,
                                                          const float* part) {
    __shared__ double red[4];
    float* x = h + (size_t)blockIdx.x * ldh;
    float4 v[NV];
    uint2 wv[NV];
    float4 p[NV][NS > 0 ? NS : 1];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int k = (threadIdx.x + 256 * i) * 4;
        v[i] = k < dim ? *reinterpret_cast<const float4*>(x + k) : float4{0.f, 0.f, 0.f, 0.f};
        wv[i] = k < dim ? *reinterpret_cast<const uint2*>(w + k) : uint2{0u, 0u};
#pragma unroll
        for (int sp = 0; sp < NS; ++sp)
            p[i][sp] = k < dim ? *reinterpret_cast<const float4*>(part + ((size_t)sp * gridDim.x + blockIdx.x) * dim + k)
                               : float4{0.f, 0.f, 0.f, 0.f};
    }
    if (NS > 0) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float4 t = p[i][0];
#pragma unroll
            for (int sp = 1; sp < NS; ++sp) {
                t.x += p[i][sp].x; t.y += p[i][sp].y; t.z += p[i][sp].z; t.w += p[i][sp].w;
            }
            v[i].x += t.x; v[i].y += t.y; v[i].z += t.z; v[i].w += t.w;
            const int k = (threadIdx.x + 256 * i) * 4;
            if (k < dim) *reinterpret_cast<float4*>(x + k) = v[i];
        }
    }
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < NV; ++i) ss += sq64(v[i].x) + sq64(v[i].y) + sq64(v[i].z) + sq64(v[i].w);
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float den = sqrtf((float)((red[0] + red[1] + red[2] + red[3]) / (double)dim) + eps);
    const float rcp = 1.0f / den;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int k = (threadIdx.x + 256 * i) * 4;
        if (k >= dim) continue;
        uint2 p;
        p.x = Mma<T16>::pack2(div_rn(v[i].x, den, rcp) * Elem<T16>::lo(wv[i].x),
                              div_rn(v[i].y, den, rcp) * Elem<T16>::hi(wv[i].x));
        p.y = Mma<T16>::pack2(div_rn(v[i].z, den, rcp) * Elem<T16>::lo(wv[i].y),
                              div_rn(v[i].w, den, rcp) * Elem<T16>::hi(wv[i].y));
        const size_t o = frag_mt ? frag_index(blockIdx.x, k, frag_mt) : (size_t)blockIdx.x * ldo + k;
        *reinterpret_cast<uint2*>(out + o) = p;
    }
}

// Same, for rows of at most 8192 elements that first take in nsplit <= NSM K-split partials
// (the split-K residual products of short prefills: up to 16 splits of a few hundred rows).
// One 1024-thread workgroup per row, two float4 positions per thread at most; all partial
// loads of a position are issued before the first is added (splits past nsplit re-read the
// last one and are not added), so the row costs one memory round trip.  Partials are summed
// in split order and then added to h, as the reduce pass of the products does.
template <typename T16, int NSM>
__global__ __launch_bounds__(1024) void rmsnorm_fold_kernel(float* h, int64_t ldh, int dim, const T16* w,
                                                           float eps, uint16_t* out, int64_t ldo, int frag_mt,
                                                           const float* part, int nsplit) {
    __shared__ double red[16];
    const int rows = gridDim.x, row = blockIdx.x;
    float* x = h + (size_t)row * ldh;
    float4 v[2];
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int k = (threadIdx.x + 1024 * i) * 4;
        v[i] = float4{0.f, 0.f, 0.f, 0.f};
        if (k < dim) {
            float4 q[NSM];
#pragma unroll
            for (int sp = 0; sp < NSM; ++sp) {
                const int z = min(sp, nsplit - 1);
                q[sp] = *reinterpret_cast<const float4*>(part + ((size_t)z * rows + row) * dim + k);
            }
            float4 hv = *reinterpret_cast<const float4*>(x + k);
            float4 t = q[0];
#pragma unroll
            for (int sp = 1; sp < NSM; ++sp) {
                if (sp < nsplit) {
                    t.x += q[sp].x; t.y += q[sp].y; t.z += q[sp].z; t.w += q[sp].w;
                }
            }
            hv.x += t.x; hv.y += t.y; hv.z += t.z; hv.w += t.w;
            *reinterpret_cast<float4*>(x + k) = hv;
            v[i] = hv;
        }
        ss += sq64(v[i].x) + sq64(v[i].y) + sq64(v[i].z) + sq64(v[i].w);
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int wv = 0; wv < 16; ++wv) tot += red[wv];
    const float den = sqrtf((float)(tot / (double)dim) + eps);
    const float rcp = 1.0f / den;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int k = (threadIdx.x + 1024 * i) * 4;
        if (k >= dim) continue;
        const uint2 wv = *reinterpret_cast<const uint2*>(w + k);
        uint2 p;
        p.x = Mma<T16>::pack2(div_rn(v[i].x, den, rcp) * Elem<T16>::lo(wv.x),
                              div_rn(v[i].y, den, rcp) * Elem<T16>::hi(wv.x));
        p.y = Mma<T16>::pack2(div_rn(v[i].z, den, rcp) * Elem<T16>::lo(wv.y),
                              div_rn(v[i].w, den, rcp) * Elem<T16>::hi(wv.y));
        const size_t o = frag_mt ? frag_index(row, k, frag_mt) : (size_t)row * ldo + k;
        *reinterpret_cast<uint2*>(out + o) = p;
    }
}

// Better of two (value, index) candidates: larger value wins, ties -> lower index, NaN never wins.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
    if (i2 < 0) return;
    if (i < 0 || v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

// One 1024-thread workgroup per row; 16-byte loads when the row is 16-byte aligned.
__global__ __launch_bounds__(1024) void argmax_kernel(const float* logits, int vocab, int64_t stride,
                                                      int32_t* out) {
    __shared__ float sv[16];
    __shared__ int si[16];
    const float* x = logits + (size_t)blockIdx.x * stride;
    float best = 0.f;
    int bi = -1;
    const bool vec = ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
    int k0 = 0;
    if (vec) {
        const int n4 = vocab / 4;
        for (int i = threadIdx.x; i < n4; i += 1024) {
            const float4 v = reinterpret_cast<const float4*>(x)[i];
            if (v.x == v.x) argmax_merge(best, bi, v.x, 4 * i);
            if (v.y == v.y) argmax_merge(best, bi, v.y, 4 * i + 1);
            if (v.z == v.z) argmax_merge(best, bi, v.z, 4 * i + 2);
            if (v.w == v.w) argmax_merge(best, bi, v.w, 4 * i + 3);
        }
        k0 = n4 * 4;
    }
    for (int k = k0 + threadIdx.x; k < vocab; k += 1024) {
        const float v = x[k];
        if (v == v) argmax_merge(best, bi, v, k);   // skips NaN
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float v2 = __shfl_xor(best, o, kWave);
        const int i2 = __shfl_xor(bi, o, kWave);
        argmax_merge(best, bi, v2, i2);
    }
    if ((threadIdx.x & 63) == 0) {
        sv[threadIdx.x >> 6] = best;
        si[threadIdx.x >> 6] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 16; ++w) argmax_merge(best, bi, sv[w], si[w]);
        out[blockIdx.x] = bi;
    }
}

__global__ void clear_flag_kernel(int32_t* flag) { *flag = 0; }

__global__ void set_step_kernel(StepState* st, int pos, int64_t ld, const int32_t* tokens,
                                float* logits) {
    st->pos = pos;
    st->pad = 0;
    st->ld = ld;
    st->tokens = tokens;
    st->logits = logits;
}

__global__ void select_kernel(const int32_t* next, int32_t* tokens, int64_t ld, int cur_pos,
                              const int32_t* prompt_len, int bsz) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < bsz && cur_pos >= prompt_len[b]) tokens[(size_t)b * ld + cur_pos] = next[b];
}

// RoPE + bf16 storage of q and the K/V cache append from fp32 projections y [T][nq+2nk]
// (used when the [wq;wk;wv] GEMM stores plainly).  One thread per (row, pair).
template <typename T16>
__global__ void rope_scatter_kernel(const float* y, int splits, int64_t ldy, int T, QkvTarget t) {
    const int npairs = (t.nq + 2 * t.nk) / 2;
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)T * npairs) return;
    const int m = (int)(i / npairs);
    const int n0 = 2 * (int)(i - (size_t)m * npairs);
    float y0 = 0.f, y1 = 0.f;
    for (int z = 0; z < splits; ++z) {     // partial projections, summed in split order
        const float2 v = *reinterpret_cast<const float2*>(y + ((size_t)z * T + m) * ldy + n0);
        y0 += v.x;
        y1 += v.y;
    }
    const int mm = t.row0 + m;             // row of the bsz x seqlen rectangle
    const int b = mm / t.seqlen;
    const int pos = t.start_pos + (mm - b * t.seqlen);
    if (n0 < t.nq + t.nk) {
        const float2 cs = t.rope[(size_t)pos * (t.head_dim / 2) + (n0 % t.head_dim) / 2];
        const float r0 = y0 * cs.x - y1 * cs.y;
        const float r1 = y0 * cs.y + y1 * cs.x;
        y0 = r0;
        y1 = r1;
    }
    if (n0 < t.nq) {
        *reinterpret_cast<float2*>(t.q + (size_t)mm * t.nq + n0) = make_float2(Mma<T16>::round(y0), Mma<T16>::round(y1));
        return;
    }
    const bool is_k = n0 < t.nq + t.nk;
    const int c = is_k ? n0 - t.nq : n0 - t.nq - t.nk;
    uint16_t* cache = static_cast<uint16_t*>(is_k ? t.cache_k : t.cache_v);
    *reinterpret_cast<uint32_t*>(cache + ((size_t)b * t.max_seq + pos) * (size_t)t.nk + c) = Mma<T16>::pack2(y0, y1);
}

}  // namespace

hipError_t launch_rope_scatter_parts(const float* y, int splits, int64_t ldy, int T, const QkvTarget& t,
                                     hipStream_t s, int wtype) {
    const size_t n = (size_t)T * ((t.nq + 2 * t.nk) / 2);
    const dim3 grid((unsigned)((n + 255) / 256));
    if (wtype == kStoreBf16)
        launch_kernel(rope_scatter_kernel<bf16>, grid, dim3(256), 0, s, y, splits, ldy, T, t);
    else if (wtype == kStoreF16)
        launch_kernel(rope_scatter_kernel<f16>, grid, dim3(256), 0, s, y, splits, ldy, T, t);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}


hipError_t launch_embed(const int32_t* tokens, int64_t ld, int bsz, int seqlen, const void* table,
                        int wtype, int vocab, int dim, float* h, const StepState* st, hipStream_t s,
                        int32_t* err) {
    const dim3 grid(bsz * seqlen), block(256);
    switch (wtype) {
        case kStoreBf16:
            launch_kernel(embed_kernel<bf16>, grid, block, 0, s, tokens, ld, seqlen,
                          static_cast<const bf16*>(table), vocab, dim, h, st, err);
            break;
        case kStoreF16:
            launch_kernel(embed_kernel<f16>, grid, block, 0, s, tokens, ld, seqlen,
                          static_cast<const f16*>(table), vocab, dim, h, st, err);
            break;
        case kStoreF32:
            launch_kernel(embed_kernel<float>, grid, block, 0, s, tokens, ld, seqlen,
                          static_cast<const float*>(table), vocab, dim, h, st, err);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_clear_flag(int32_t* flag, hipStream_t s) {
    launch_kernel(clear_flag_kernel, dim3(1), dim3(1), 0, s, flag);
    return hipGetLastError();
}

hipError_t launch_set_step(StepState* st, int pos, int64_t ld, const int32_t* tokens, float* logits,
                           hipStream_t s) {
    launch_kernel(set_step_kernel, dim3(1), dim3(1), 0, s, st, pos, ld, tokens, logits);
    return hipGetLastError();
}

template <typename T16, int NS>
void launch_rmsnorm_ns(float* h, int64_t ldh, int rows, int dim, const T16* wb, float eps, uint16_t* o,
                       int64_t ldo, int frag_mt, const float* part, hipStream_t s) {
    switch ((dim + 1023) / 1024) {
        case 1: launch_kernel((rmsnorm_reg_kernel<T16, 1, NS>), dim3(rows), dim3(256), 0, s, h, ldh, dim, wb, eps, o, ldo, frag_mt, part); break;
        case 2: launch_kernel((rmsnorm_reg_kernel<T16, 2, NS>), dim3(rows), dim3(256), 0, s, h, ldh, dim, wb, eps, o, ldo, frag_mt, part); break;
        case 3:
        case 4: launch_kernel((rmsnorm_reg_kernel<T16, 4, NS>), dim3(rows), dim3(256), 0, s, h, ldh, dim, wb, eps, o, ldo, frag_mt, part); break;
        case 5:
        case 6: launch_kernel((rmsnorm_reg_kernel<T16, 6, NS>), dim3(rows), dim3(256), 0, s, h, ldh, dim, wb, eps, o, ldo, frag_mt, part); break;
        default: launch_kernel((rmsnorm_reg_kernel<T16, 8, NS>), dim3(rows), dim3(256), 0, s, h, ldh, dim, wb, eps, o, ldo, frag_mt, part); break;
    }
}

template <typename T16>
void launch_rmsnorm16(float* h, int64_t ldh, int rows, int dim, const void* w, float eps, uint16_t* o, int64_t ldo,
                      int frag_mt, hipStream_t s, const float* part, int nsplit) {
    const T16* wb = static_cast<const T16*>(w);
    if (nsplit > 2 && dim <= 8192) {
        if (nsplit <= 4)
            launch_kernel((rmsnorm_fold_kernel<T16, 4>), dim3(rows), dim3(1024), 0, s, h, ldh, dim, wb, eps, o, ldo,
                          frag_mt, part, nsplit);
        else if (nsplit <= 8)
            launch_kernel((rmsnorm_fold_kernel<T16, 8>), dim3(rows), dim3(1024), 0, s, h, ldh, dim, wb, eps, o, ldo,
                          frag_mt, part, nsplit);
        else
            launch_kernel((rmsnorm_fold_kernel<T16, 16>), dim3(rows), dim3(1024), 0, s, h, ldh, dim, wb, eps, o, ldo,
                          frag_mt, part, nsplit);
    } else if (dim > 8192 || nsplit > 2)
        launch_kernel(rmsnorm_bf16_kernel<T16>, dim3(rows), dim3(256), 0, s, h, ldh, dim, wb, eps, o, ldo, frag_mt,
                      part, nsplit);
    else if (nsplit == 2)
        launch_rmsnorm_ns<T16, 2>(h, ldh, rows, dim, wb, eps, o, ldo, frag_mt, part, s);
    else
        launch_rmsnorm_ns<T16, 0>(h, ldh, rows, dim, wb, eps, o, ldo, frag_mt, nullptr, s);
}

hipError_t launch_rmsnorm_bf16(float* h, int64_t ldh, int rows, int dim, const void* w,
                               float eps, void* out, int64_t ldo, int frag_mt, hipStream_t s,
                               const float* part, int nsplit, int wtype) {
    uint16_t* o = static_cast<uint16_t*>(out);
    if (nsplit > 1 && (!part || nsplit > kMaxNormFold)) return hipErrorInvalidValue;
    if (wtype == kStoreBf16)
        launch_rmsnorm16<bf16>(h, ldh, rows, dim, w, eps, o, ldo, frag_mt, s, part, nsplit);
    else if (wtype == kStoreF16)
        launch_rmsnorm16<f16>(h, ldh, rows, dim, w, eps, o, ldo, frag_mt, s, part, nsplit);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, int bsz, int vocab, int64_t stride, int32_t* out,
                         hipStream_t s) {
    launch_kernel(argmax_kernel, dim3(bsz), dim3(1024), 0, s, logits, vocab, stride, out);
    return hipGetLastError();
}

hipError_t launch_select(const int32_t* next, int32_t* tokens, int64_t ld, int cur_pos,
                         const int32_t* prompt_len, int bsz, hipStream_t s) {
    launch_kernel(select_kernel, dim3((bsz + 63) / 64), dim3(64), 0, s, next, tokens, ld,
                       cur_pos, prompt_len, bsz);
    return hipGetLastError();
}

}  // namespace llk
