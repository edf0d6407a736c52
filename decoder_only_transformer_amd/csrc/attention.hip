// Causal grouped-query attention of individual query rows against the KV cache
// (flash-decode style).  One workgroup handles one query position, one kv head and all
// n_rep query heads that read it (GQA without materialising repeat_kv), over one split of
// the visible keys [0, pos].  Sixteen lanes share one key (head_dim/16 elements each); each
// 16-lane group loads four keys' K and V rows before using any of them and keeps a running
// (max, sum, acc) online softmax per head in fp32.  The sixteen groups are merged through
// LDS.  With more than one split per row, every workgroup stores its partial (m, l, acc)
// with device-coherent stores and the last one to arrive (per-row counter) merges all
// splits in split order and resets the counter, so no second launch is needed and the
// result is deterministic.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kMaxSplitMerge = 32;   // largest split count the in-kernel merge handles

// N elements of a K or V row as raw bits (4, 8, 16 or 32 bytes), unpacked later so the
// loads of several keys are in flight together.
template <typename KT, int N>
struct RawRow {
    static constexpr int kWords = N * (int)sizeof(KT) / 4;
    uint32_t w[kWords];
    __device__ __forceinline__ void load(const KT* p) {
        if constexpr (kWords == 8) {
            const uint4 a = ld16(p), b = ld16(reinterpret_cast<const char*>(p) + 16);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
        } else if constexpr (kWords == 4) {
            const uint4 a = ld16(p);
            w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        } else if constexpr (kWords == 2) {
            const uint2 a = *reinterpret_cast<const uint2*>(p);
            w[0] = a.x; w[1] = a.y;
        } else {
            w[0] = *reinterpret_cast<const uint32_t*>(p);
        }
    }
    __device__ __forceinline__ void unpack(float* out) const {
        if constexpr (sizeof(KT) == 4) {
#pragma unroll
            for (int i = 0; i < N; ++i) out[i] = __uint_as_float(w[i]);
        } else {
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                out[2 * i] = bf16lo(w[i]);
                out[2 * i + 1] = bf16hi(w[i]);
            }
        }
    }
};



// Merge running softmax state (m, l, acc) with the one held by lane ^ `o`.
template <int NREP, int EPL>
__device__ __forceinline__ void merge_with_lane(float (&m)[NREP], float (&l)[NREP],
                                                float (&acc)[NREP][EPL], int o) {
#pragma unroll
    for (int r = 0; r < NREP; ++r) {
        const float mo = __shfl_xor(m[r], o, kWave);
        const float lo = __shfl_xor(l[r], o, kWave);
        const float M = fmaxf(m[r], mo);
        const float a1 = (M == -INFINITY) ? 0.f : __expf(m[r] - M);
        const float a2 = (M == -INFINITY) ? 0.f : __expf(mo - M);
        l[r] = l[r] * a1 + lo * a2;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const float ao = __shfl_xor(acc[r][e], o, kWave);
            acc[r][e] = acc[r][e] * a1 + ao * a2;
        }
        m[r] = M;
    }
}

template <typename KT, int HD, int NREP, bool OUT_BF16, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void attn_rows_kernel(AttnArgs a) {
    constexpr int EPL = HD / 16;
    constexpr int SLOTS = WAVES * 4;     // 16-lane groups, one key each at a time
    constexpr int PF = 4;                // keys per group whose loads are in flight together
    __shared__ float s_m[WAVES][NREP];
    __shared__ float s_l[WAVES][NREP];
    __shared__ float s_acc[WAVES][NREP][HD];

    const int split = blockIdx.x, kvh = blockIdx.y, t = a.row0 + blockIdx.z;
    const int b = t / a.seqlen;
    const int start_pos = a.st ? a.st->pos : a.start_pos;
    const int pos = start_pos + (t - b * a.seqlen);
    const int ctx = pos + 1;
    // keys per split: given, or (graph replay) derived from this step's context as the host
    // would: ceil(ctx / n_split) rounded up to 16
    const int chunk = a.chunk ? a.chunk : ((start_pos + a.seqlen + a.n_split - 1) / a.n_split + 15) / 16 * 16;
    const int j0 = split * chunk;
    const int j1 = min(ctx, j0 + chunk);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int grp = lane >> 4, gl = lane & 15;
    const int slot = wid * 4 + grp;
    const int qstride = a.n_heads * HD;
    const int64_t kv_row = (int64_t)a.n_kv_heads * HD;

    const size_t base = (size_t)b * a.max_seq * kv_row + (size_t)kvh * HD + gl * EPL;
    const KT* kb = static_cast<const KT*>(a.cache_k) + base;
    const KT* vb = static_cast<const KT*>(a.cache_v) + base;

    // q stays unscaled; 1/sqrt(hd) is applied to each score.  Its loads are independent of
    // the K/V loads below and complete under them.
    float q[NREP][EPL];
#pragma unroll
    for (int r = 0; r < NREP; ++r)
#pragma unroll
        for (int e = 0; e < EPL; ++e)
            q[r][e] = a.q[(size_t)t * qstride + (kvh * NREP + r) * HD + gl * EPL + e];

    float m[NREP], l[NREP], acc[NREP][EPL];
#pragma unroll
    for (int r = 0; r < NREP; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[r][e] = 0.f;
    }

    for (int j = j0 + slot; j < j1; j += PF * SLOTS) {
        RawRow<KT, EPL> kr[PF], vr[PF];
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int jj = min(j + u * SLOTS, j1 - 1);   // clamped: unconditional loads
            kr[u].load(kb + (size_t)jj * kv_row);
            vr[u].load(vb + (size_t)jj * kv_row);
        }
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            if (j + u * SLOTS >= j1) break;
            float kf[EPL], vf[EPL];
            kr[u].unpack(kf);
            vr[u].unpack(vf);
#pragma unroll
            for (int r = 0; r < NREP; ++r) {
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) s += q[r][e] * kf[e];
                s = group_sum<16>(s) * a.scale;
                const float mn = fmaxf(m[r], s);
                const float sc = __expf(m[r] - mn);
                const float p = __expf(s - mn);
                l[r] = l[r] * sc + p;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[r][e] = acc[r][e] * sc + p * vf[e];
                m[r] = mn;
            }
        }
    }

    // the four 16-lane groups of a wave hold the same d range: merge them by shuffles
    merge_with_lane<NREP, EPL>(m, l, acc, 16);
    merge_with_lane<NREP, EPL>(m, l, acc, 32);
    if (grp == 0) {
#pragma unroll
        for (int r = 0; r < NREP; ++r) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) s_acc[wid][r][gl * EPL + e] = acc[r][e];
            if (gl == 0) {
                s_m[wid][r] = m[r];
                s_l[wid][r] = l[r];
            }
        }
    }
    __syncthreads();

    for (int idx = tid; idx < NREP * HD; idx += blockDim.x) {
        const int r = idx / HD, d = idx - r * HD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_m[w][r]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < WAVES; ++w) {
                const float wt = __expf(s_m[w][r] - M);
                L += s_l[w][r] * wt;
                A += s_acc[w][r][d] * wt;
            }
        }
        const int h = kvh * NREP + r;
        if (a.n_split == 1) {
            const float o = A / L;
            if (OUT_BF16)
                static_cast<uint16_t*>(a.out)[a.out_frag_mt ? frag_index(t, h * HD + d, a.out_frag_mt)
                                                            : (size_t)t * qstride + h * HD + d] = f32_to_bf16(o);
            else
                static_cast<float*>(a.out)[(size_t)t * qstride + h * HD + d] = o;
        } else {
            float* pp = a.part + (((size_t)t * a.n_heads + h) * a.n_split + split) * (HD + 2);
            st_agent(pp + d, A);
            if (d == 0) {
                st_agent(pp + HD, M);
                st_agent(pp + HD + 1, L);
            }
        }
    }
    if (a.n_split == 1) return;

    // Last workgroup of this (row, kv head) to arrive merges the splits; the partials went
    // out as device-coherent stores and are read back the same way.
    __shared__ int s_last;
    int* counter = &a.counters[(size_t)t * a.n_kv_heads + kvh];
    if (!arrive_last(counter, a.n_split, &s_last)) return;
    for (int idx = tid; idx < NREP * HD; idx += blockDim.x) {
        const int r = idx / HD, d = idx - r * HD;
        const int h = kvh * NREP + r;
        const float* pp = a.part + ((size_t)t * a.n_heads + h) * a.n_split * (HD + 2);
        float ms[kMaxSplitMerge], ls[kMaxSplitMerge], as[kMaxSplitMerge];
        float M = -INFINITY;
#pragma unroll
        for (int sp = 0; sp < kMaxSplitMerge; ++sp) {
            if (sp < a.n_split) {
                ms[sp] = ld_agent(pp + sp * (HD + 2) + HD);
                ls[sp] = ld_agent(pp + sp * (HD + 2) + HD + 1);
                as[sp] = ld_agent(pp + sp * (HD + 2) + d);
                M = fmaxf(M, ms[sp]);
            }
        }
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int sp = 0; sp < kMaxSplitMerge; ++sp) {
            if (sp < a.n_split && ms[sp] != -INFINITY) {
                const float w = __expf(ms[sp] - M);
                L += ls[sp] * w;
                A += as[sp] * w;
            }
        }
        const float o = A / L;
        if (OUT_BF16)
            static_cast<uint16_t*>(a.out)[a.out_frag_mt ? frag_index(t, h * HD + d, a.out_frag_mt)
                                                        : (size_t)t * qstride + h * HD + d] = f32_to_bf16(o);
        else
            static_cast<float*>(a.out)[(size_t)t * qstride + h * HD + d] = o;
    }
    if (tid == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waves per workgroup: many for single-token rows (decode: one workgroup covers a short
// context in one round of loads), four for prefill rows; capped so that the per-lane state
// of NREP heads fits the register budget.
template <int NREP> constexpr int kDecodeWaves = NREP <= 2 ? 16 : 8;

template <typename KT, int HD, int NREP, bool OB>
hipError_t launch4(const AttnArgs& args, hipStream_t s) {
    constexpr int kMaxZ = 65535;
    for (int r0 = 0; r0 < args.rows; r0 += kMaxZ) {
        AttnArgs a = args;
        a.row0 = r0;
        const int n = min(kMaxZ, args.rows - r0);
        const dim3 grid(a.n_split, a.n_kv_heads, n);
        if (a.seqlen == 1)
            launch_kernel((attn_rows_kernel<KT, HD, NREP, OB, kDecodeWaves<NREP>>), grid,
                               dim3(64 * kDecodeWaves<NREP>), 0, s, a);
        else
            launch_kernel((attn_rows_kernel<KT, HD, NREP, OB, 4>), grid, dim3(256), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
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
