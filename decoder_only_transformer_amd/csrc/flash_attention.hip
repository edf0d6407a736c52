// Causal grouped-query attention for prefill on 16-bit MFMA (gfx950 v_mfma_f32_16x16x32_bf16,
// or _f16 for fp16 models: every kernel takes the storage type T16 of q, the cache and the
// output).
//
// A workgroup owns one batch row, one kv head and 128 query rows, a query row being a
// (position, head) pair of the n_rep heads that read this kv head (GQA is never
// materialised: the K/V tile in LDS serves all of them).  Four waves own 32 rows each, as
// two 16-row tiles that share every K and V fragment read.
// K/V advance in tiles of 64 keys up to the last position any row of the workgroup sees; the
// next tile's loads are in flight while the current tile is computed.
//
//  S^T = K Q^T    keys are the MFMA M dimension, so after the product each lane holds
//                 4 consecutive keys of one query; per-query max and sum need only two
//                 cross-lane steps (lanes l, l^16, l^32, l^48 share a query).
//  O^T += V^T P^T the K dimension of this product is taken in a permuted order: lane group
//                 g feeds keys {4g..4g+3} of the first 16-key half and {16+4g..16+4g+3} of
//                 the second, exactly the 8 scores the lane already holds, so P never moves
//                 between lanes.  V is staged transposed in LDS to match.
//  P is split into a 16-bit high part and a 16-bit remainder (two MFMAs), so the weights keep
//  ~16 (bf16) or ~22 (fp16) significant bits and the attention is computed with fp32-softmax
//  semantics; Q, K and V are 16-bit tensors already (stored so by the projection).  With fp16,
//  p <= 2^8 (see the running max below) stays far inside the format's range; a p below 2^-24 of
//  the row maximum flushes to zero, below fp32's resolution of the row sum.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));

constexpr int kRows = 128;    // query rows per workgroup: 4 waves x 2 tiles of 16
constexpr int kQT = 2;        // 16-row query tiles per wave (each K/V fragment read feeds both)

// Position of key `key` (0..63) of a tile in a V^T row: each 32-key half is stored in the
// permuted k order of the O^T product, so lane group g's 8 keys {4g..4g+3, 16+4g..16+4g+3}
// are one contiguous 16-byte read.
__device__ __forceinline__ int vt_pos(int key) {
    const int half = key & ~31, r = key & 31;
    return half + ((r & 15) >> 2) * 8 + (r >> 4) * 4 + (r & 3);
}
constexpr int kKeys = 64;     // keys per tile

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Two floats to two round-to-nearest-even 16-bit values in one word (low half = a); bf16 with
// gfx950's paired conversion.
template <typename T16>
__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
    if constexpr (std::is_same<T16, bf16>::value)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2_t));
    else
        return Mma<T16>::pack2(a, b);
}

template <typename T16, int HD>
__global__ __launch_bounds__(256, 2) void flash_prefill_kernel(FlashArgs a) {
    typedef typename Mma<T16>::v8 v8_t;
    constexpr int KS = HD / 32;            // MFMA k-steps over head_dim
    constexpr int DT = HD / 16;            // 16-row tiles of head_dim in O^T
    constexpr int KLD = HD + 8;            // padded K row (elements)
    constexpr int VLD = kKeys + 8;         // padded V^T row (elements)
    constexpr int CH = HD / 8;                   // 16-byte chunks per key row
    constexpr int CPT = kKeys * CH / 256;        // chunks per thread per tile
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kKeys][KLD];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][HD][VLD];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int fr = lane & 15, g = lane >> 4;
    // Workgroup -> (batch row, kv head, query tile).  The dispatcher deals workgroup ids
    // round-robin over the 8 XCDs; ids are mapped so each XCD gets a contiguous run of
    // (pair, tile), i.e. all query tiles of a (row, kv head) pair run on one XCD and share its
    // K/V through that XCD's L2.  Within a pair the longest tiles (most keys) go first.
    const int n_qt = (a.seqlen * (a.n_heads / a.n_kv_heads) + kRows - 1) / kRows;
    const int total = n_qt * a.n_kv_heads * a.bsz;
    const int per_xcd = (total + 7) / 8;
    const int lin = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
    if (lin >= total) return;
    const int pair = lin / n_qt;
    const int qtile = n_qt - 1 - (lin - pair * n_qt);
    const int kvh = pair % a.n_kv_heads, b = pair / a.n_kv_heads;
    const int n_rep = a.n_heads / a.n_kv_heads;
    const int qstride = a.n_heads * HD;
    const int64_t kv_row = (int64_t)a.n_kv_heads * HD;

    // Query rows of the workgroup: the tiles end at the last row, so when the rows are not a
    // whole number of tiles the partial tile is the first one (rows -pad .. kRows - pad - 1),
    // which sees the fewest keys.
    const int pad = n_qt * kRows - a.seqlen * n_rep;

    // Keys visible to the workgroup: up to the largest position among its rows.
    const int last_row = qtile * kRows + kRows - 1 - pad;
    const int kend = a.start_pos + last_row / n_rep + 1;     // exclusive
    const int first_row = max(qtile * kRows - pad, 0);
    const int kfull = a.start_pos + first_row / n_rep + 1;   // keys < kfull are visible to all rows

    const uint16_t* kbase = static_cast<const uint16_t*>(a.cache_k) + (size_t)b * a.max_seq * kv_row + (size_t)kvh * HD;
    const uint16_t* vbase = static_cast<const uint16_t*>(a.cache_v) + (size_t)b * a.max_seq * kv_row + (size_t)kvh * HD;

    // K/V tiles of 64 keys: the next tile's loads are in flight (registers) while the current
    // one is computed from LDS; two LDS buffers, one barrier per tile.
    uint4 kreg[CPT], vreg[CPT];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + 256 * i;
            const int key = c % kKeys, d8 = (c / kKeys) * 8;   // key-fastest: V^T stores spread over banks
            const int kk = min(k0 + key, kend - 1);   // clamp: rows past kend are masked anyway
            kreg[i] = ld16(kbase + (size_t)kk * kv_row + d8);
            vreg[i] = ld16(vbase + (size_t)kk * kv_row + d8);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int c = tid + 256 * i;
            const int key = c % kKeys, d8 = (c / kKeys) * 8;
            *reinterpret_cast<uint4*>(&Ks[buf][key][d8]) = kreg[i];
            const uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                Vt[buf][d8 + 2 * q][vt_pos(key)] = static_cast<uint16_t>(w[q] & 0xffffu);
                Vt[buf][d8 + 2 * q + 1][vt_pos(key)] = static_cast<uint16_t>(w[q] >> 16);
            }
        }
    };

    // the first K/V tile is in flight while the Q fragments load
    if (kend > 0) load_tile(0);

    // This lane's query rows: column fr of the wave's S^T tiles qt = 0, 1.  Rows before the
    // prompt (in a partial first tile) compute with the first position's keys and are not
    // stored.
    int s_idx[kQT], head[kQT], qpos[kQT];
    bool row_ok[kQT];
    v8_t qf[kQT][KS];
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
        const int r_raw = qtile * kRows + wid * 16 * kQT + qt * 16 + fr - pad;
        row_ok[qt] = r_raw >= 0;
        const int r_local = row_ok[qt] ? r_raw : 0;
        s_idx[qt] = r_local / n_rep;                       // position within the prompt
        head[qt] = kvh * n_rep + r_local % n_rep;
        qpos[qt] = a.start_pos + s_idx[qt];                // absolute position
        // Q fragments (fp32 holding 16-bit values in the q buffer -> exact conversion)
        const float* qp = a.q + ((size_t)b * a.seqlen + s_idx[qt]) * qstride + head[qt] * HD;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u16x8_t v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = Mma<T16>::bits(qp[ks * 32 + g * 8 + e]);
            qf[qt][ks] = __builtin_bit_cast(v8_t, v);
        }
    }

    // Online softmax in base 2: with c2 = scale * log2(e), p = 2^(s c2 - m).  The
    // running max m is raised (and O, l rescaled) only when some row's tile max exceeds it by
    // more than 8, so p <= 2^8 between raises; the final O / l is the same quotient.
    const float c2 = a.scale * 1.4426950408889634f;
    float m[kQT], l[kQT];
    f32x4 o[kQT][DT];
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
        m[qt] = -INFINITY;
        l[qt] = 0.f;
#pragma unroll
        for (int t = 0; t < DT; ++t) o[qt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int k0 = 0, it = 0; k0 < kend; k0 += kKeys, ++it) {
        const int buf = it & 1;
        store_tile(buf);
        __syncthreads();
        if (k0 + kKeys < kend) load_tile(k0 + kKeys);

        // ---- S^T for 4 key tiles of 16: lane holds keys k0 + 16j + 4g + e of query column fr.
        //      The K fragments of key tile j + 1 are read while the MFMAs of tile j run.
        f32x4 st[kQT][4];
        v8_t kf[2][KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[0][ks] = *reinterpret_cast<const v8_t*>(&Ks[buf][fr][ks * 32 + g * 8]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < 3) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kf[(j + 1) & 1][ks] = *reinterpret_cast<const v8_t*>(&Ks[buf][16 * (j + 1) + fr][ks * 32 + g * 8]);
            }
#pragma unroll
            for (int qt = 0; qt < kQT; ++qt) st[qt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int qt = 0; qt < kQT; ++qt)
                    st[qt][j] = Mma<T16>::mma(kf[j & 1][ks], qf[qt][ks], st[qt][j]);
        }
        // first V fragment of the O^T product, read while the softmax runs
        v8_t vf[2];
        vf[0] = *reinterpret_cast<const v8_t*>(&Vt[buf][fr][8 * g]);
        // ---- causal mask (tiles reaching past the first row's position only), online softmax
        //      per query (= per lane column; lanes l, l^16, l^32, l^48 share one).  The row
        //      maximum is taken over the raw scores; the scale enters the exponent through one
        //      FMA: p = 2^(s c2 - m).
        const bool diag = k0 + kKeys > kfull;
        u32x4_t phi[kQT][2], plo[kQT][2];
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt) {
            float tmax = -INFINITY;
            if (diag) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = k0 + 16 * j + 4 * g + e;
                        const float v = key > qpos[qt] ? -INFINITY : st[qt][j][e];
                        st[qt][j][e] = v;
                        tmax = fmaxf(tmax, v);
                    }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, st[qt][j][e]);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
            tmax *= c2;
            if (__any(tmax > m[qt] + 8.f)) {
                const float mn = fmaxf(m[qt], tmax);
                const float alpha = __builtin_amdgcn_exp2f(m[qt] - mn);   // 0 on the first tile
                l[qt] *= alpha;
#pragma unroll
                for (int t = 0; t < DT; ++t) o[qt][t] *= alpha;
                m[qt] = mn;
            }
            float psum = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; e += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[qt][j][e], c2, -m[qt]));
                    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[qt][j][e + 1], c2, -m[qt]));
                    psum += p0 + p1;
                    // P = hi + lo, both 16-bit; k-slot of key (j, e) in the permuted PV order:
                    // half kk = j / 2, slot (j % 2) * 4 + e of the lane group's 8
                    const uint32_t hi = cvt_pk<T16>(p0, p1);
                    const uint32_t lo = cvt_pk<T16>(p0 - Mma<T16>::value(static_cast<uint16_t>(hi & 0xffffu)),
                                                    p1 - Mma<T16>::value(static_cast<uint16_t>(hi >> 16)));
                    phi[qt][j >> 1][(j & 1) * 2 + e / 2] = hi;
                    plo[qt][j >> 1][(j & 1) * 2 + e / 2] = lo;
                }
            psum += __shfl_xor(psum, 16, kWave);
            psum += __shfl_xor(psum, 32, kWave);
            l[qt] += psum;
        }

        // ---- O^T += V^T P^T over the two 32-key halves (permuted k order); fragment i + 1 is
        //      read while the MFMAs of fragment i run
#pragma unroll
        for (int i = 0; i < 2 * DT; ++i) {
            const int kk = i / DT, t = i % DT;
            if (i + 1 < 2 * DT) {
                const int kn = (i + 1) / DT, tn = (i + 1) % DT;
                // the 8 keys of lane group g in this half, already in k-slot order
                vf[(i + 1) & 1] = *reinterpret_cast<const v8_t*>(&Vt[buf][16 * tn + fr][32 * kn + 8 * g]);
            }
#pragma unroll
            for (int qt = 0; qt < kQT; ++qt) {
                o[qt][t] = Mma<T16>::mma(vf[i & 1], __builtin_bit_cast(v8_t, phi[qt][kk]), o[qt][t]);
                o[qt][t] = Mma<T16>::mma(vf[i & 1], __builtin_bit_cast(v8_t, plo[qt][kk]), o[qt][t]);
            }
        }
    }

    // ---- O = O^T / l, stored 16-bit at [b*seqlen + s][head*hd + d]: 4 consecutive d per store
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
        if (!row_ok[qt]) continue;
        const float inv = 1.f / l[qt];
        uint16_t* out = static_cast<uint16_t*>(a.out) + ((size_t)b * a.seqlen + s_idx[qt]) * qstride + head[qt] * HD;
#pragma unroll
        for (int t = 0; t < DT; ++t) {
            uint2 w;
            w.x = cvt_pk<T16>(o[qt][t][0] * inv, o[qt][t][1] * inv);
            w.y = cvt_pk<T16>(o[qt][t][2] * inv, o[qt][t][3] * inv);
            *reinterpret_cast<uint2*>(out + 16 * t + 4 * g) = w;
        }
    }
}

}  // namespace

hipError_t launch_flash_prefill(const FlashArgs& a, hipStream_t s) {
    const int n_rep = a.n_heads / a.n_kv_heads;
    const int n_qt = (a.seqlen * n_rep + kRows - 1) / kRows;
    const int total = n_qt * a.n_kv_heads * a.bsz;
    const dim3 grid((unsigned)((total + 7) / 8 * 8));     // padded: bijective XCD mapping
    const bool f16 = a.wtype == kStoreF16;
    if (!f16 && a.wtype != kStoreBf16) return hipErrorInvalidValue;
    if (a.head_dim == 128)
        launch_kernel(f16 ? flash_prefill_kernel<llk::f16, 128> : flash_prefill_kernel<bf16, 128>, grid, dim3(256), 0, s, a);
    else if (a.head_dim == 64)
        launch_kernel(f16 ? flash_prefill_kernel<llk::f16, 64> : flash_prefill_kernel<bf16, 64>, grid, dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace llk
