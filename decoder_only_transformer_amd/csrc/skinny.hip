// Weight-streaming products for a few activation rows on bf16 MFMA (decode with batch > 4).
//
// y[m][n] = sum_k x[m][k] * W[n][k] for M <= 32 rows.  The vector-ALU GEMV would spend M FMAs
// per weight element; here the weights are the MFMA A operand instead: a workgroup owns 16
// output rows (16 hidden units for the SiLU gate, from w1 and w3), its four waves take
// interleaved 32-wide k-steps, each lane streams 16 bytes of one weight row per k-step with
// eight k-steps of loads in flight, and the activations -- bf16 [M][K], L2 resident -- are
// read directly as B fragments (rows of the batch as MFMA columns).  The waves' partial
// sums meet in LDS; the result tile D[n][m] puts the RoPE pair (n, n+1) in one lane.
// Epilogues match the GEMV ones: RoPE + bf16 q / KV append, residual add, SiLU gate (bf16
// out), fp32 logits.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kPF = 8;        // k-steps of weight loads in flight per wave

__device__ __forceinline__ bf16x8_t frag(const uint4& v) {
    return __builtin_bit_cast(bf16x8_t, u32x4_t{v.x, v.y, v.z, v.w});
}

template <int MT, int EPI>
__global__ __launch_bounds__(256) void skinny_kernel(SkinnyArgs a) {
    constexpr int NW = (EPI == EPI_SWIGLU) ? 2 : 1;    // weight matrices per output unit
    __shared__ f32x4 red[kWaves][NW][MT][64];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int fr = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int K = a.K;
    const int nsteps = K / 32;

    // weight rows of this lane (row n0 + fr of each matrix; clamped past N)
    const uint16_t* wrow[NW];
    {
        const int n = min(n0 + fr, a.N - 1);
        if (EPI == EPI_SWIGLU) {
            wrow[0] = static_cast<const uint16_t*>(a.w0) + (size_t)n * K;
            wrow[1] = static_cast<const uint16_t*>(a.w1) + (size_t)n * K;
        } else if (EPI == EPI_QKV) {
            const int nq = a.qkv.nq, nk = a.qkv.nk;
            const uint16_t* m = static_cast<const uint16_t*>(n < nq ? a.w0 : (n < nq + nk ? a.w1 : a.w2));
            const int r = n < nq ? n : (n < nq + nk ? n - nq : n - nq - nk);
            wrow[0] = m + (size_t)r * K;
        } else {
            wrow[0] = static_cast<const uint16_t*>(a.w0) + (size_t)n * K;
        }
    }
    // activation rows of this lane (batch rows fr and 16 + fr; clamped past M, masked later)
    const uint16_t* xrow[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
        xrow[t] = static_cast<const uint16_t*>(a.x) + (size_t)min(16 * t + fr, a.M - 1) * a.ldx;

    f32x4 acc[NW][MT];
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[w][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // this wave's k-steps: wid, wid + 4, ...; weight loads kPF steps ahead
    for (int s0 = wid; s0 < nsteps; s0 += kWaves * kPF) {
        uint4 wv[kPF][NW];
        uint4 xv[kPF][MT];
#pragma unroll
        for (int u = 0; u < kPF; ++u) {
            const int st = min(s0 + u * kWaves, nsteps - 1);
            const int k = st * 32 + g * 8;
#pragma unroll
            for (int w = 0; w < NW; ++w) wv[u][w] = ld16_stream(wrow[w] + k);
#pragma unroll
            for (int t = 0; t < MT; ++t) xv[u][t] = ld16(xrow[t] + k);
        }
        asm volatile("" ::: "memory");   // keep all kPF steps of loads issued before any use
#pragma unroll
        for (int u = 0; u < kPF; ++u) {
            // steps past the end were loaded clamped; a zero weight fragment cancels them
            const bool live = s0 + u * kWaves < nsteps;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const uint4 wz = live ? wv[u][w] : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[w][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag(wz), frag(xv[u][t]), acc[w][t], 0, 0, 0);
            }
        }
    }

    // sum the four waves' partials
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int t = 0; t < MT; ++t) red[wid][w][t][lane] = acc[w][t];
    __syncthreads();
    if (wid != 0) return;
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            f32x4 v = red[0][w][t][lane];
#pragma unroll
            for (int q = 1; q < kWaves; ++q) v += red[q][w][t][lane];
            acc[w][t] = v;
        }

    // lane holds D[n = n0 + 4g + e][m = 16t + fr]
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int m = 16 * t + fr;
        if (m >= a.M) continue;
        if (EPI == EPI_QKV) {
            const QkvTarget& q = a.qkv;
            const int b = m / q.seqlen;
            const int pos = (q.st ? q.st->pos : q.start_pos) + (m - b * q.seqlen);
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
                const int n = n0 + 4 * g + e;
                if (n >= a.N) continue;
                float y0 = acc[0][t][e], y1 = acc[0][t][e + 1];
                if (n < q.nq + q.nk) {
                    const float2 cs = q.rope[(size_t)pos * (q.head_dim / 2) + (n % q.head_dim) / 2];
                    const float r0 = y0 * cs.x - y1 * cs.y;
                    const float r1 = y0 * cs.y + y1 * cs.x;
                    y0 = r0;
                    y1 = r1;
                }
                if (n < q.nq) {
                    q.q[(size_t)m * q.nq + n] = round_bf16(y0);
                    q.q[(size_t)m * q.nq + n + 1] = round_bf16(y1);
                } else {
                    const bool is_k = n < q.nq + q.nk;
                    const int c = is_k ? n - q.nq : n - q.nq - q.nk;
                    uint16_t* cache = static_cast<uint16_t*>(is_k ? q.cache_k : q.cache_v);
                    *reinterpret_cast<uint32_t*>(cache + ((size_t)b * q.max_seq + pos) * (size_t)q.nk + c) =
                        pack_bf16x2(y0, y1);
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = n0 + 4 * g + e;
                if (n >= a.N) continue;
                if (EPI == EPI_RESID) {
                    a.resid[(size_t)m * a.ldr + n] += acc[0][t][e];
                } else if (EPI == EPI_SWIGLU) {
                    static_cast<uint16_t*>(a.out16)[(size_t)m * a.ldo + n] =
                        f32_to_bf16(silu(acc[0][t][e]) * acc[NW - 1][t][e]);
                } else {
                    (a.st ? a.st->logits : a.out)[(size_t)m * a.ldo + n] = acc[0][t][e];
                }
            }
        }
    }
}

template <int EPI>
hipError_t launch_epi(const SkinnyArgs& a, hipStream_t s) {
    const dim3 grid((a.N + 15) / 16);
    if (a.M <= 16)
        launch_kernel((skinny_kernel<1, EPI>), grid, dim3(256), 0, s, a);
    else
        launch_kernel((skinny_kernel<2, EPI>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_skinny(int epi, const SkinnyArgs& a, hipStream_t s) {
    if (a.M > 32 || a.K % 32 != 0) return hipErrorInvalidValue;
    switch (epi) {
        case EPI_QKV: return launch_epi<EPI_QKV>(a, s);
        case EPI_RESID: return launch_epi<EPI_RESID>(a, s);
        case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(a, s);
        default: return launch_epi<EPI_STORE>(a, s);
    }
}

}  // namespace llk
