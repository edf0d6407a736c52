// Causal grouped-query attention of individual query rows against the KV cache
// (flash-decode style).  One workgroup handles one query position, one kv head and all
// n_rep query heads that read it (GQA without materialising repeat_kv), over one split of
// the visible keys [0, pos].  Sixteen lanes share one key (head_dim/16 elements each), a
// wave walks four keys at a time, and each 16-lane group keeps a running (max, sum, acc)
// online softmax per head in fp32.  The sixteen groups are merged through LDS; with more
// than one split per row a second kernel merges the per-split partials.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kSlots = 16;   // 4 waves x 4 lane groups

template <typename KT, int N>
__device__ __forceinline__ void load_row(const KT* p, float* out) {
    constexpr int bytes = N * (int)sizeof(KT);
    if constexpr (bytes == 32) {
        Elem<KT>::unpack(ld16(p), out);
        Elem<KT>::unpack(ld16(p + 16 / sizeof(KT)), out + 16 / sizeof(KT));
    } else if constexpr (bytes == 16) {
        Elem<KT>::unpack(ld16(p), out);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) out[i] = Elem<KT>::load(p, i);
    }
}

template <typename KT, int HD, int NREP, bool OUT_BF16>
__global__ __launch_bounds__(256) void attn_rows_kernel(AttnArgs a) {
    constexpr int EPL = HD / 16;
    __shared__ float s_m[kSlots][NREP];
    __shared__ float s_l[kSlots][NREP];
    __shared__ float s_acc[kSlots][NREP][HD];

    const int split = blockIdx.x, kvh = blockIdx.y, t = a.row0 + blockIdx.z;
    const int b = t / a.seqlen;
    const int pos = a.start_pos + (t - b * a.seqlen);
    const int ctx = pos + 1;
    const int j0 = split * a.chunk;
    const int j1 = min(ctx, j0 + a.chunk);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int grp = lane >> 4, gl = lane & 15;
    const int slot = wid * 4 + grp;
    const int qstride = a.n_heads * HD;
    const int64_t kv_row = (int64_t)a.n_kv_heads * HD;

    float q[NREP][EPL];
#pragma unroll
    for (int r = 0; r < NREP; ++r)
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            q[r][e] = a.q[(size_t)t * qstride + (kvh * NREP + r) * HD + gl * EPL + e] * a.scale;

    float m[NREP], l[NREP], acc[NREP][EPL];
#pragma unroll
    for (int r = 0; r < NREP; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[r][e] = 0.f;
    }

    const size_t base = (size_t)b * a.max_seq * kv_row + (size_t)kvh * HD + gl * EPL;
    const KT* kb = static_cast<const KT*>(a.cache_k) + base;
    const KT* vb = static_cast<const KT*>(a.cache_v) + base;
    for (int j = j0 + slot; j < j1; j += kSlots) {
        float kf[EPL], vf[EPL];
        load_row<KT, EPL>(kb + (size_t)j * kv_row, kf);
        load_row<KT, EPL>(vb + (size_t)j * kv_row, vf);
#pragma unroll
        for (int r = 0; r < NREP; ++r) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) s += q[r][e] * kf[e];
            s = group_sum<16>(s);
            const float mn = fmaxf(m[r], s);
            const float sc = __expf(m[r] - mn);
            const float p = __expf(s - mn);
            l[r] = l[r] * sc + p;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[r][e] = acc[r][e] * sc + p * vf[e];
            m[r] = mn;
        }
    }

#pragma unroll
    for (int r = 0; r < NREP; ++r) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_acc[slot][r][gl * EPL + e] = acc[r][e];
        if (gl == 0) {
            s_m[slot][r] = m[r];
            s_l[slot][r] = l[r];
        }
    }
    __syncthreads();

    for (int idx = tid; idx < NREP * HD; idx += blockDim.x) {
        const int r = idx / HD, d = idx - r * HD;
        float M = -INFINITY;
#pragma unroll
        for (int sl = 0; sl < kSlots; ++sl) M = fmaxf(M, s_m[sl][r]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int sl = 0; sl < kSlots; ++sl) {
                const float w = __expf(s_m[sl][r] - M);
                L += s_l[sl][r] * w;
                A += s_acc[sl][r][d] * w;
            }
        }
        const int h = kvh * NREP + r;
        if (a.n_split == 1) {
            const float o = A / L;
            if (OUT_BF16)
                static_cast<uint16_t*>(a.out)[(size_t)t * qstride + h * HD + d] = f32_to_bf16(o);
            else
                static_cast<float*>(a.out)[(size_t)t * qstride + h * HD + d] = o;
        } else {
            float* pp = a.part + (((size_t)t * a.n_heads + h) * a.n_split + split) * (HD + 2);
            pp[d] = A;
            if (d == 0) {
                pp[HD] = M;
                pp[HD + 1] = L;
            }
        }
    }
}

template <int HD, bool OUT_BF16>
__global__ void attn_merge_kernel(AttnArgs a) {
    const int t = a.row0 + blockIdx.x, h = blockIdx.y, d = threadIdx.x;
    const float* pp = a.part + ((size_t)t * a.n_heads + h) * a.n_split * (HD + 2);
    float M = -INFINITY;
    for (int s = 0; s < a.n_split; ++s) M = fmaxf(M, pp[s * (HD + 2) + HD]);
    float L = 0.f, A = 0.f;
    for (int s = 0; s < a.n_split; ++s) {
        const float ms = pp[s * (HD + 2) + HD];
        if (ms == -INFINITY) continue;
        const float w = __expf(ms - M);
        L += pp[s * (HD + 2) + HD + 1] * w;
        A += pp[s * (HD + 2) + d] * w;
    }
    const float o = A / L;
    const size_t idx = (size_t)t * a.n_heads * HD + h * HD + d;
    if (OUT_BF16)
        static_cast<uint16_t*>(a.out)[idx] = f32_to_bf16(o);
    else
        static_cast<float*>(a.out)[idx] = o;
}

template <typename KT, int HD, int NREP, bool OB>
hipError_t launch4(const AttnArgs& args, hipStream_t s) {
    constexpr int kMaxZ = 65535;
    for (int r0 = 0; r0 < args.rows; r0 += kMaxZ) {
        AttnArgs a = args;
        a.row0 = r0;
        const int n = min(kMaxZ, args.rows - r0);
        hipLaunchKernelGGL((attn_rows_kernel<KT, HD, NREP, OB>), dim3(a.n_split, a.n_kv_heads, n),
                           dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (a.n_split > 1) {
            hipLaunchKernelGGL((attn_merge_kernel<HD, OB>), dim3(n, a.n_heads), dim3(HD), 0, s, a);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

template <typename KT, int HD, bool OB>
hipError_t launch3(const AttnArgs& a, hipStream_t s) {
    switch (a.n_heads / a.n_kv_heads) {
        case 1: return launch4<KT, HD, 1, OB>(a, s);
        case 2: return launch4<KT, HD, 2, OB>(a, s);
        case 4: return launch4<KT, HD, 4, OB>(a, s);
        case 8: return launch4<KT, HD, 8, OB>(a, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename KT, bool OB>
hipError_t launch2(const AttnArgs& a, hipStream_t s) {
    switch (a.head_dim) {
        case 32: return launch3<KT, 32, OB>(a, s);
        case 64: return launch3<KT, 64, OB>(a, s);
        case 128: return launch3<KT, 128, OB>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_attn_rows(int kv_bf16, const AttnArgs& a, hipStream_t s) {
    if (kv_bf16) return a.out_bf16 ? launch2<bf16, true>(a, s) : launch2<bf16, false>(a, s);
    return a.out_bf16 ? launch2<float, true>(a, s) : launch2<float, false>(a, s);
}

}  // namespace llk
