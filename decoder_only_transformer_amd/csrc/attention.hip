// Causal grouped-query attention of individual query rows against the KV cache
// (flash-decode style).  One workgroup handles one query position, one kv head and all
// n_rep query heads that read it (GQA without materialising repeat_kv), over one split of
// the visible keys [0, pos].  Sixteen lanes share one key (head_dim/16 elements each); each
// 16-lane group loads four keys' K and V rows before using any of them and keeps a running
// (max, sum, acc) online softmax per head in fp32.  The sixteen groups are merged through
// LDS.  With more than one split per row, every workgroup stores its partial (m, l, acc)
// and a second, small launch combines the splits in split order (deterministic; the kernel
// boundary makes the partials visible without any cross-workgroup synchronisation).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace llk {
namespace {


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
                out[2 * i] = Elem<KT>::lo(w[i]);
                out[2 * i + 1] = Elem<KT>::hi(w[i]);
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

// A 16-bit output in the cache's storage type: fp16 for fp16 caches, bf16 otherwise.
template <typename KT>
__device__ __forceinline__ uint16_t out16(float x) {
    if constexpr (std::is_same<KT, f16>::value)
        return f32_to_f16(x);
    else
        return f32_to_bf16(x);
}

// Second pass of a split launch: output (row t, head h, dim d) from the n_split partials
// (m, l, acc) of its splits, combined in split order.  One workgroup per (row, head), one
// thread per dim; the partials were written by the first pass with plain stores.
template <typename KT, bool OUT_BF16>
__global__ __launch_bounds__(128) void attn_merge_kernel(AttnArgs a) {
    const int t = a.row0 + blockIdx.y, h = blockIdx.x, d = threadIdx.x;
    const int HD = a.head_dim;
    if (d >= HD) return;
    const float* pp = a.part + ((size_t)t * a.n_heads + h) * a.n_split * (HD + 2);
    float M = -INFINITY;
    for (int sp = 0; sp < a.n_split; ++sp) M = fmaxf(M, pp[sp * (HD + 2) + HD]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
        for (int sp = 0; sp < a.n_split; ++sp) {
            const float m = pp[sp * (HD + 2) + HD];
            if (m == -INFINITY) continue;
            const float w = __expf(m - M);
            L += pp[sp * (HD + 2) + HD + 1] * w;
            A += pp[sp * (HD + 2) + d] * w;
        }
    }
    const float o = A / L;
    const size_t qstride = (size_t)a.n_heads * HD;
    if (OUT_BF16)
        static_cast<uint16_t*>(a.out)[a.out_frag_mt ? frag_index(t, h * HD + d, a.out_frag_mt)
                                                    : (size_t)t * qstride + h * HD + d] = out16<KT>(o);
    else
        static_cast<float*>(a.out)[(size_t)t * qstride + h * HD + d] = o;
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
                                                            : (size_t)t * qstride + h * HD + d] = out16<KT>(o);
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

// ---------------------------------------------------------------------------------------
// Decode rows with several query heads per kv head (GQA, n_rep >= 4) on MFMA.  The n_rep
// query heads of one position share every K/V row, so per workgroup (row, kv head, key
// split) the scores are a small matrix product: S^T = K Q^T (16x16x32 MFMA, keys as rows,
// the n_rep heads as columns padded to 16) and O^T += V^T P^T (16x16x16 MFMA).  A lane of
// S^T holds 4 consecutive keys of one head, which is exactly the B fragment P^T needs, so
// the probabilities never move between lanes; P is split into a bf16 high part and a bf16
// remainder (two MFMAs) to keep fp32-softmax accuracy.  K (row-major) and V^T tiles of 64
// keys are staged in LDS, double-buffered, with one barrier per tile; each of the four waves
// takes 16 keys of a tile and keeps its own online-softmax state, merged at the end through
// LDS.  Splits are combined by the merge pass.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8v __attribute__((ext_vector_type(8)));

template <int HD, int NREP, bool OUT_BF16>
__global__ __launch_bounds__(256) void attn_gqa_decode_kernel(AttnArgs a) {
    constexpr int KT = 64;             // keys per tile, 16 per wave
    constexpr int KS = HD / 32;        // k-steps of S^T over head_dim
    constexpr int DT = HD / 16;        // 16-row tiles of O^T
    constexpr int KLD = HD + 8;        // padded K row (elements)
    constexpr int VLD = KT + 8;        // padded V^T row (elements)
    constexpr int CH = KT * HD / 8;    // 16-byte chunks of a K (or V) tile
    constexpr int CPT = CH / 256;      // chunks per thread
    static_assert(NREP <= 16 && CPT >= 1, "shape");
    // staging buffers; after the last tile the same memory holds the waves' O^T for the merge
    constexpr int kStageBytes = 2 * KT * KLD * 2 + 2 * HD * VLD * 2;
    constexpr int kMergeBytes = 4 * HD * 17 * 4;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kStageBytes > kMergeBytes ? kStageBytes : kMergeBytes];
    auto Ks = reinterpret_cast<uint16_t(*)[KT][KLD]>(lds);
    auto Vt = reinterpret_cast<uint16_t(*)[HD][VLD]>(lds + 2 * KT * KLD * 2);
    auto s_o = reinterpret_cast<float(*)[HD][17]>(lds);
    __shared__ float s_m[4][16], s_l[4][16];

    const int split = blockIdx.x, kvh = blockIdx.y, t = a.row0 + blockIdx.z;
    const int b = t / a.seqlen;
    const int start_pos = a.st ? a.st->pos : a.start_pos;
    const int pos = start_pos + (t - b * a.seqlen);
    const int ctx = pos + 1;
    const int chunk = a.chunk ? a.chunk : ((start_pos + a.seqlen + a.n_split - 1) / a.n_split + 15) / 16 * 16;
    const int j0 = split * chunk;
    const int j1 = min(ctx, j0 + chunk);
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int fr = lane & 15, g = lane >> 4;
    const int qstride = a.n_heads * HD;
    const int64_t kv_row = (int64_t)a.n_kv_heads * HD;
    const uint16_t* kbase = static_cast<const uint16_t*>(a.cache_k) + (size_t)b * a.max_seq * kv_row + (size_t)kvh * HD;
    const uint16_t* vbase = static_cast<const uint16_t*>(a.cache_v) + (size_t)b * a.max_seq * kv_row + (size_t)kvh * HD;

    // Q^T fragments: column fr = head kvh * NREP + fr (zero past NREP), k = 32 ks + 8 g + e
    bf16x8v qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u16x8v v;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            v[e] = fr < NREP ? f32_to_bf16(a.q[(size_t)t * qstride + (kvh * NREP + fr) * HD + ks * 32 + g * 8 + e]) : 0;
        qf[ks] = __builtin_bit_cast(bf16x8v, v);
    }

    // staging: chunk c of a tile is key c % KT, dims (c / KT) * 8 .. + 7 (key-fastest, so the
    // V^T stores of a wave spread over banks)
    // two tiles of loads in flight: register sets R = 0, 1 hold tiles it and it + 1 while
    // tile it - 1 is computed
    uint4 kreg[2][CPT], vreg[2][CPT];
    auto load_tile = [&](int k0, int R) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + 256 * i;
            const int key = c % KT, d8 = (c / KT) * 8;
            const int kk = min(k0 + key, j1 - 1);          // clamped: masked below
            kreg[R][i] = ld16(kbase + (size_t)kk * kv_row + d8);
            vreg[R][i] = ld16(vbase + (size_t)kk * kv_row + d8);
        }
    };
    auto store_tile = [&](int buf, int R) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + 256 * i;
            const int key = c % KT, d8 = (c / KT) * 8;
            *reinterpret_cast<uint4*>(&Ks[buf][key][d8]) = kreg[R][i];
            const uint32_t w[4] = {vreg[R][i].x, vreg[R][i].y, vreg[R][i].z, vreg[R][i].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                Vt[buf][d8 + 2 * q][key] = static_cast<uint16_t>(w[q] & 0xffffu);
                Vt[buf][d8 + 2 * q + 1][key] = static_cast<uint16_t>(w[q] >> 16);
            }
        }
    };

    float m = -INFINITY, l = 0.f;       // online softmax of head fr over this wave's keys
    f32x4v o[DT];
#pragma unroll
    for (int d = 0; d < DT; ++d) o[d] = f32x4v{0.f, 0.f, 0.f, 0.f};

    const int n_tiles = (j1 - j0 + KT - 1) / KT;
    if (n_tiles > 0) load_tile(j0, 0);
    if (n_tiles > 1) load_tile(j0 + KT, 1);
    auto tile_step = [&](int it, int buf) {   // buf = it & 1 = register set of tile it
        const int k0 = j0 + it * KT;
        store_tile(buf, buf);
        __syncthreads();
        if (it + 2 < n_tiles) load_tile(k0 + 2 * KT, buf);   // in flight under two tiles' products

        // S^T for keys k0 + 16 wid + (4g + e), head fr
        f32x4v st = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8v kf = *reinterpret_cast<const bf16x8v*>(&Ks[buf][16 * wid + fr][ks * 32 + g * 8]);
            st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], st, 0, 0, 0);
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = k0 + 16 * wid + 4 * g + e;
            st[e] = key < j1 ? st[e] * a.scale : -INFINITY;
            tmax = fmaxf(tmax, st[e]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
        const float mn = fmaxf(m, tmax);
        const float alpha = (mn == -INFINITY) ? 1.f : __expf(m - mn);
        float psum = 0.f;
        s16x4 phi, plo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p = (mn == -INFINITY) ? 0.f : __expf(st[e] - mn);
            psum += p;
            const uint16_t hi = f32_to_bf16(p);
            phi[e] = static_cast<short>(hi);
            plo[e] = static_cast<short>(f32_to_bf16(p - bf16_to_f32(hi)));
        }
        psum += __shfl_xor(psum, 16, kWave);
        psum += __shfl_xor(psum, 32, kWave);
        l = l * alpha + psum;
        m = mn;
        // O^T[dims 16 d + 4 g + e][head fr] += V^T[dim][keys 16 wid + 4 g' + j] P^T
#pragma unroll
        for (int d = 0; d < DT; ++d) {
            o[d] *= alpha;
            const s16x4 vf = *reinterpret_cast<const s16x4*>(&Vt[buf][16 * d + fr][16 * wid + 4 * g]);
            o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, phi, o[d], 0, 0, 0);
            o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, plo, o[d], 0, 0, 0);
        }
    };
    for (int it = 0; it < n_tiles; it += 2) {
        tile_step(it, 0);
        if (it + 1 < n_tiles) tile_step(it + 1, 1);
    }

    // merge the four waves: lane (fr, g) holds O^T[16 d + 4 g + e][fr]
    __syncthreads();                                  // every wave is done with the last tile
    if (g == 0) {
        s_m[wid][fr] = m;
        s_l[wid][fr] = l;
    }
#pragma unroll
    for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int e = 0; e < 4; ++e) s_o[wid][16 * d + 4 * g + e][fr] = o[d][e];
    __syncthreads();

    for (int idx = tid; idx < NREP * HD; idx += 256) {
        const int r = idx / HD, d = idx - r * HD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, s_m[w][r]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float wt = __expf(s_m[w][r] - M);
                L += s_l[w][r] * wt;
                A += s_o[w][d][r] * wt;
            }
        }
        const int h = kvh * NREP + r;
        if (a.n_split == 1) {
            const float ov = A / L;
            if (OUT_BF16)
                static_cast<uint16_t*>(a.out)[a.out_frag_mt ? frag_index(t, h * HD + d, a.out_frag_mt)
                                                            : (size_t)t * qstride + h * HD + d] = f32_to_bf16(ov);
            else
                static_cast<float*>(a.out)[(size_t)t * qstride + h * HD + d] = ov;
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
        bool done = false;
        if constexpr (NREP >= 4 && std::is_same<KT, bf16>::value) {
            if (a.seqlen == 1) {
                launch_kernel((attn_gqa_decode_kernel<HD, NREP, OB>), grid, dim3(256), 0, s, a);
                done = true;
            }
        }
        if (done) {
        } else if (a.seqlen == 1 && NREP == 1 && n * a.n_kv_heads >= 512)
            // many (row, head) pairs, each a workgroup: 4 waves, so that all of them are
            // resident at once (16-wave workgroups would leave a partial second round)
            launch_kernel((attn_rows_kernel<KT, HD, NREP, OB, 4>), grid, dim3(256), 0, s, a);
        else if (a.seqlen == 1)
            launch_kernel((attn_rows_kernel<KT, HD, NREP, OB, kDecodeWaves<NREP>>), grid,
                               dim3(64 * kDecodeWaves<NREP>), 0, s, a);
        else
            launch_kernel((attn_rows_kernel<KT, HD, NREP, OB, 4>), grid, dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (a.n_split > 1) {
            launch_kernel((attn_merge_kernel<KT, OB>), dim3(a.n_heads, n), dim3(128), 0, s, a);
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

hipError_t launch_attn_rows(int kv_type, const AttnArgs& a, hipStream_t s) {
    switch (kv_type) {
        case kStoreBf16: return a.out_bf16 ? launch2<bf16, true>(a, s) : launch2<bf16, false>(a, s);
        case kStoreF32: return a.out_bf16 ? launch2<float, true>(a, s) : launch2<float, false>(a, s);
        // fp16 caches: fp32 output on the vector path; 16-bit (fp16) output for the MFMA
        // products' operand
        case kStoreF16: return a.out_bf16 ? launch2<f16, true>(a, s) : launch2<f16, false>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace llk
