// Weight-streaming matrix-vector products on the vector ALUs (gfx950, wave64).
//
// y[m][n] = sum_k x[m][k] * W[n][k] for a handful of activation rows m (decode: one row per
// batch entry) against an nn.Linear-oriented weight W [N][K].  The work is bound by reading
// W from HBM once, so each wave owns two output columns (two weight rows), every lane keeps
// up to 16 independent 16-byte weight loads in flight, and the activations -- optionally
// RMS-normalised on the fly (fused attention_norm / ffn_norm / final norm) -- are staged
// once per workgroup in LDS as fp32.  Epilogues fuse what follows each projection in the
// block: RoPE + KV-cache append for [wq; wk; wv], residual add for wo / w2, the SiLU gate
// for [w1; w3], and the fp32 logits store for the output projection.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kSeg = 4096;   // activation elements staged per LDS segment

template <typename WT>
__device__ __forceinline__ const WT* qkv_row(const GemvArgs& a, int n) {
    const int nq = a.qkv.nq, nk = a.qkv.nk;
    if (n < nq) return static_cast<const WT*>(a.w0) + (size_t)n * a.K;
    if (n < nq + nk) return static_cast<const WT*>(a.w1) + (size_t)(n - nq) * a.K;
    return static_cast<const WT*>(a.w2) + (size_t)(n - nq - nk) * a.K;
}

// RoPE for a pair (y0, y1) = (x[2i], x[2i+1]) at `pos`, then store q / K / V.
template <typename WT>
__device__ __forceinline__ void qkv_store(const QkvTarget& t, int m, int n0, float y0, float y1) {
    const int b = m / t.seqlen;
    const int pos = t.start_pos + m % t.seqlen;
    const int hd = t.head_dim;
    if (n0 < t.nq + t.nk) {
        const float2 cs = t.rope[(size_t)pos * (hd / 2) + (n0 % hd) / 2];
        const float r0 = y0 * cs.x - y1 * cs.y;
        const float r1 = y0 * cs.y + y1 * cs.x;
        y0 = r0;
        y1 = r1;
    }
    if (n0 < t.nq) {
        t.q[(size_t)m * t.nq + n0] = y0;
        t.q[(size_t)m * t.nq + n0 + 1] = y1;
        return;
    }
    const bool is_k = n0 < t.nq + t.nk;
    const int c = is_k ? n0 - t.nq : n0 - t.nq - t.nk;     // kv_head*hd + d
    WT* cache = static_cast<WT*>(is_k ? t.cache_k : t.cache_v);
    const size_t off = ((size_t)b * t.max_seq + pos) * (size_t)t.nk + c;
    Elem<WT>::store(cache, off, y0);
    Elem<WT>::store(cache, off + 1, y1);
}

template <typename WT, int MB, int EPI, bool NORM>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a) {
    constexpr int VEC = Elem<WT>::kPer16B;
    constexpr int U = 8;
    __shared__ float xs[MB][kSeg];
    __shared__ float red[kWavesPerBlock][MB];
    __shared__ float rstd_s[MB];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid >> 6;
    const int unit = blockIdx.x * kWavesPerBlock + wid;
    const int n_units = (EPI == EPI_SWIGLU) ? a.N : a.N / 2;
    const bool active = unit < n_units;

    // The two weight rows this wave streams.
    const WT* row0 = nullptr;
    const WT* row1 = nullptr;
    int n0 = 0;
    if (active) {
        if (EPI == EPI_SWIGLU) {
            n0 = unit;
            row0 = static_cast<const WT*>(a.w0) + (size_t)unit * a.K;
            row1 = static_cast<const WT*>(a.w1) + (size_t)unit * a.K;
        } else if (EPI == EPI_QKV) {
            n0 = 2 * unit;
            row0 = qkv_row<WT>(a, n0);
            row1 = row0 + a.K;
        } else {
            n0 = 2 * unit;
            row0 = static_cast<const WT*>(a.w0) + (size_t)n0 * a.K;
            row1 = row0 + a.K;
        }
    }

    for (int m0 = 0; m0 < a.M; m0 += MB) {
        if (NORM) {
            float ss[MB];
#pragma unroll
            for (int m = 0; m < MB; ++m) ss[m] = 0.f;
            for (int k = tid * 4; k < a.K; k += kThreads * 4) {
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    if (m0 + m < a.M) {
                        const float4 v = *reinterpret_cast<const float4*>(a.x + (size_t)(m0 + m) * a.ldx + k);
                        ss[m] += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                const float t = wave_sum(ss[m]);
                if (lane == 0) red[wid][m] = t;
            }
            __syncthreads();
            if (tid < MB) {
                float t = 0.f;
                for (int w = 0; w < kWavesPerBlock; ++w) t += red[w][tid];
                rstd_s[tid] = rsqrtf(t / (float)a.K + a.eps);
            }
            __syncthreads();
        }

        float acc[MB][2];
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[m][0] = acc[m][1] = 0.f;

        for (int k0 = 0; k0 < a.K; k0 += kSeg) {
            const int klen = min(kSeg, a.K - k0);
            __syncthreads();
            for (int i = tid; i < MB * (klen / 4); i += kThreads) {
                const int m = i / (klen / 4);
                const int k = (i - m * (klen / 4)) * 4;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                if (m0 + m < a.M) {
                    v = *reinterpret_cast<const float4*>(a.x + (size_t)(m0 + m) * a.ldx + k0 + k);
                    if (NORM) {
                        const WT* nw = static_cast<const WT*>(a.norm_w) + k0 + k;
                        const float r = rstd_s[m];
                        v.x = v.x * r * Elem<WT>::load(nw, 0);
                        v.y = v.y * r * Elem<WT>::load(nw, 1);
                        v.z = v.z * r * Elem<WT>::load(nw, 2);
                        v.w = v.w * r * Elem<WT>::load(nw, 3);
                    }
                }
                *reinterpret_cast<float4*>(&xs[m][k]) = v;
            }
            __syncthreads();
            if (active) {
                const int nchunks = klen / VEC;
                const WT* p0 = row0 + k0;
                const WT* p1 = row1 + k0;
                for (int c = lane; c < nchunks; c += kWave * U) {
                    uint4 w0v[U], w1v[U];
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int cc = c + kWave * u;
                        if (cc < nchunks) {
                            w0v[u] = ld16_stream(p0 + (size_t)cc * VEC);
                            w1v[u] = ld16_stream(p1 + (size_t)cc * VEC);
                        }
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int cc = c + kWave * u;
                        if (cc < nchunks) {
                            float f0[VEC], f1[VEC];
                            Elem<WT>::unpack(w0v[u], f0);
                            Elem<WT>::unpack(w1v[u], f1);
#pragma unroll
                            for (int m = 0; m < MB; ++m) {
                                const float* xp = &xs[m][cc * VEC];
#pragma unroll
                                for (int j = 0; j < VEC; j += 4) {
                                    const float4 xv = *reinterpret_cast<const float4*>(xp + j);
                                    acc[m][0] += f0[j] * xv.x + f0[j + 1] * xv.y + f0[j + 2] * xv.z + f0[j + 3] * xv.w;
                                    acc[m][1] += f1[j] * xv.x + f1[j + 1] * xv.y + f1[j + 2] * xv.z + f1[j + 3] * xv.w;
                                }
                            }
                        }
                    }
                }
            }
        }

        if (active) {
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                acc[m][0] = wave_sum(acc[m][0]);
                acc[m][1] = wave_sum(acc[m][1]);
            }
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                const int row = m0 + m;
                if (lane == m && row < a.M) {
                    const float y0 = acc[m][0], y1 = acc[m][1];
                    if (EPI == EPI_QKV) {
                        qkv_store<WT>(a.qkv, row, n0, y0, y1);
                    } else if (EPI == EPI_RESID) {
                        float* r = a.resid + (size_t)row * a.ldr + n0;
                        r[0] += y0;
                        r[1] += y1;
                    } else if (EPI == EPI_SWIGLU) {
                        a.out[(size_t)row * a.ldo + n0] = silu(y0) * y1;
                    } else {
                        float* o = a.out + (size_t)row * a.ldo + n0;
                        o[0] = y0;
                        o[1] = y1;
                    }
                }
            }
        }
    }
}

template <typename WT, int EPI, bool NORM>
hipError_t launch_mb(const GemvArgs& a, hipStream_t s) {
    const int n_units = (EPI == EPI_SWIGLU) ? a.N : a.N / 2;
    const dim3 grid((n_units + kWavesPerBlock - 1) / kWavesPerBlock);
    if (a.M == 1) {
        hipLaunchKernelGGL((gemv_kernel<WT, 1, EPI, NORM>), grid, dim3(kThreads), 0, s, a);
    } else if (a.M == 2) {
        hipLaunchKernelGGL((gemv_kernel<WT, 2, EPI, NORM>), grid, dim3(kThreads), 0, s, a);
    } else {
        hipLaunchKernelGGL((gemv_kernel<WT, 4, EPI, NORM>), grid, dim3(kThreads), 0, s, a);
    }
    return hipGetLastError();
}

template <typename WT>
hipError_t launch_typed(int epi, const GemvArgs& a, hipStream_t s) {
    const bool norm = a.norm_w != nullptr;
    switch (epi) {
        case EPI_QKV:
            return norm ? launch_mb<WT, EPI_QKV, true>(a, s) : launch_mb<WT, EPI_QKV, false>(a, s);
        case EPI_RESID:
            return norm ? launch_mb<WT, EPI_RESID, true>(a, s) : launch_mb<WT, EPI_RESID, false>(a, s);
        case EPI_SWIGLU:
            return norm ? launch_mb<WT, EPI_SWIGLU, true>(a, s) : launch_mb<WT, EPI_SWIGLU, false>(a, s);
        default:
            return norm ? launch_mb<WT, EPI_STORE, true>(a, s) : launch_mb<WT, EPI_STORE, false>(a, s);
    }
}

}  // namespace

hipError_t launch_gemv(int wbf16, int epi, const GemvArgs& a, hipStream_t s) {
    return wbf16 ? launch_typed<bf16>(epi, a, s) : launch_typed<float>(epi, a, s);
}

}  // namespace llk
