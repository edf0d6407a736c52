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
// With 16-bit weights (bf16 or fp16) the activations are rounded to that type as they are
// staged, and q is rounded before it is stored: the path stores the same 16-bit tensors as
// the MFMA prefill path (normalised operands, q, K/V, attention output, gated FFN activation).
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;


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
    const int pos = (t.st ? t.st->pos : t.start_pos) + m % t.seqlen;
    const int hd = t.head_dim;
    if (n0 < t.nq + t.nk) {
        const float2 cs = t.rope[(size_t)pos * (hd / 2) + (n0 % hd) / 2];
        const float r0 = y0 * cs.x - y1 * cs.y;
        const float r1 = y0 * cs.y + y1 * cs.x;
        y0 = r0;
        y1 = r1;
    }
    if (n0 < t.nq) {
        if (Elem<WT>::k16) {
            y0 = Elem<WT>::round(y0);
            y1 = Elem<WT>::round(y1);
        }
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

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// outstanding global loads (which __syncthreads' release fence would drain), so weight
// loads issued before it stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <typename WT, int MB, int EPI, bool NORM>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvArgs a) {
    constexpr int VEC = Elem<WT>::kPer16B;
    constexpr int U = 8;                       // 16-byte chunks per lane per row per segment
    constexpr int SEG = U * kWave * VEC;       // K elements per segment (bf16: 4096, fp32: 2048)
    constexpr int XPT = SEG / 4 / kThreads;    // activation float4s per thread per row per segment
    __shared__ float xs[MB][SEG];
    __shared__ double red[kWavesPerBlock][MB];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid >> 6;
    const int n_units = (EPI == EPI_SWIGLU) ? a.N : a.N / 2;
    const int unit_raw = blockIdx.x * kWavesPerBlock + wid;
    const bool active = unit_raw < n_units;
    // Inactive waves (tail of the last workgroup) stream a valid row and discard it, so every
    // load below is unconditional and the wait counts stay exact.
    const int unit = active ? unit_raw : n_units - 1;
    const bool one_seg = a.K <= SEG;

    const WT* row0;
    const WT* row1;
    int n0;
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

    for (int m0 = 0; m0 < a.M; m0 += MB) {
        // RMS denominators sqrt(mean(x^2) + eps): squares summed in fp64 (exact), the mean
        // rounded once to fp32, correctly rounded square root; the operand is x / den * w with
        // the correctly rounded division (div_rn, the row's reciprocal computed once).  A reciprocal times x, or a mean off by one bit,
        // differs from this in the last bit, which a 16-bit rounding of an embedding row
        // scaled onto exact ties can turn into hundreds of flipped elements.
        float den[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m) den[m] = 1.f;
        if (NORM && !one_seg) {
            // rows longer than one segment: statistics in a pass of their own
            double ss[MB];
#pragma unroll
            for (int m = 0; m < MB; ++m) ss[m] = 0.0;
            for (int k = tid * 4; k < a.K; k += kThreads * 4) {
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    const int row = min(m0 + m, a.M - 1);
                    const float4 v = *reinterpret_cast<const float4*>(a.x + (size_t)row * a.ldx + k);
                    ss[m] += sq64(v.x) + sq64(v.y) + sq64(v.z) + sq64(v.w);
                }
            }
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                const double t = wave_sum(ss[m]);
                if (lane == 0) red[wid][m] = t;
            }
            lds_barrier();
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                double t = 0.0;
#pragma unroll
                for (int w = 0; w < kWavesPerBlock; ++w) t += red[w][m];
                den[m] = sqrtf((float)(t / (double)a.K) + a.eps);
            }
            lds_barrier();
        }

        float acc[MB][2];
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[m][0] = acc[m][1] = 0.f;

        for (int k0 = 0; k0 < a.K; k0 += SEG) {
            const int klen = min(SEG, a.K - k0);
            const int nchunks = klen / VEC;
            // 1. activation (and norm weight) loads of this segment; addresses are clamped
            //    in range so every load is unconditional
            float4 xv[MB][XPT];
            uint2 nv[XPT];
            float4 nvf[XPT];
#pragma unroll
            for (int i = 0; i < XPT; ++i) {
                const int k = min((tid + i * kThreads) * 4, klen - 4);
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    const int row = min(m0 + m, a.M - 1);
                    xv[m][i] = *reinterpret_cast<const float4*>(a.x + (size_t)row * a.ldx + k0 + k);
                }
                if (NORM) {
                    if (Elem<WT>::k16)
                        nv[i] = *reinterpret_cast<const uint2*>(static_cast<const WT*>(a.norm_w) + k0 + k);
                    else
                        nvf[i] = *reinterpret_cast<const float4*>(static_cast<const WT*>(a.norm_w) + k0 + k);
                }
            }
            // 2. weight loads: in flight while the activations are normalised and staged
            uint4 w0v[U], w1v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int cc = min(lane + kWave * u, nchunks - 1);
                w0v[u] = ld16_stream(row0 + k0 + (size_t)cc * VEC);
                w1v[u] = ld16_stream(row1 + k0 + (size_t)cc * VEC);
            }
            asm volatile("" ::: "memory");   // keep the weight loads issued before the staging
            // 3. norm weights to fp32; 0/1 factors for rows past M and (for the statistics)
            //    for duplicated loads past the segment end -- arithmetic, no branches
            float kin[XPT];
#pragma unroll
            for (int i = 0; i < XPT; ++i) {
                kin[i] = (tid + i * kThreads) * 4 < klen ? 1.f : 0.f;
                if constexpr (NORM && Elem<WT>::k16)
                    nvf[i] = make_float4(Elem<WT>::lo(nv[i].x), Elem<WT>::hi(nv[i].x), Elem<WT>::lo(nv[i].y),
                                         Elem<WT>::hi(nv[i].y));
            }
            // NORM: the row's denominator and its correctly rounded reciprocal (rows past M:
            // 1 and 0, which normalise them to 0); otherwise a 1 / 0 factor
            float scale[MB], rcp[MB];
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                const bool live = m0 + m < a.M;
                scale[m] = live ? den[m] : (NORM ? 1.f : 0.f);
                rcp[m] = live ? 1.f / scale[m] : 0.f;
            }
            // 4. RMS statistics when the whole row is this segment
            if (NORM && one_seg) {
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    double ss = 0.0;
#pragma unroll
                    for (int i = 0; i < XPT; ++i)
                        ss += (double)kin[i] * (sq64(xv[m][i].x) + sq64(xv[m][i].y) + sq64(xv[m][i].z) +
                                                sq64(xv[m][i].w));
                    ss = wave_sum(ss);
                    if (lane == 0) red[wid][m] = ss;
                }
                lds_barrier();
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    double t = 0.0;
#pragma unroll
                    for (int w = 0; w < kWavesPerBlock; ++w) t += red[w][m];
                    const bool live = m0 + m < a.M;
                    scale[m] = live ? sqrtf((float)(t / (double)a.K) + a.eps) : 1.f;
                    rcp[m] = live ? 1.f / scale[m] : 0.f;
                }
            }
            // 5. normalise, round to the stored precision, stage in LDS (positions past the
            //    segment end hold duplicates and are never read)
#pragma unroll
            for (int i = 0; i < XPT; ++i) {
                const int k = (tid + i * kThreads) * 4;
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    float4 v = xv[m][i];
                    if (NORM) {
                        v.x = div_rn(v.x, scale[m], rcp[m]) * nvf[i].x;
                        v.y = div_rn(v.y, scale[m], rcp[m]) * nvf[i].y;
                        v.z = div_rn(v.z, scale[m], rcp[m]) * nvf[i].z;
                        v.w = div_rn(v.w, scale[m], rcp[m]) * nvf[i].w;
                    } else {
                        v.x *= scale[m];
                        v.y *= scale[m];
                        v.z *= scale[m];
                        v.w *= scale[m];
                    }
                    if (Elem<WT>::k16) {
                        v.x = Elem<WT>::round(v.x);
                        v.y = Elem<WT>::round(v.y);
                        v.z = Elem<WT>::round(v.z);
                        v.w = Elem<WT>::round(v.w);
                    }
                    *reinterpret_cast<float4*>(&xs[m][k]) = v;
                }
            }
            lds_barrier();
            // 6. dot products (chunks past the row end were loaded clamped and are skipped)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int cc = lane + kWave * u;
                if (cc < nchunks) {
                    float f0[VEC], f1[VEC];
                    Elem<WT>::unpack(w0v[u], f0);
                    Elem<WT>::unpack(w1v[u], f1);
#pragma unroll
                    for (int m = 0; m < MB; ++m) {
                        const float* xp = &xs[m][cc * VEC];
#pragma unroll
                        for (int j = 0; j < VEC; j += 4) {
                            const float4 xq = *reinterpret_cast<const float4*>(xp + j);
                            acc[m][0] += f0[j] * xq.x + f0[j + 1] * xq.y + f0[j + 2] * xq.z + f0[j + 3] * xq.w;
                            acc[m][1] += f1[j] * xq.x + f1[j + 1] * xq.y + f1[j + 2] * xq.z + f1[j + 3] * xq.w;
                        }
                    }
                }
            }
            lds_barrier();   // xs and red are rewritten next
        }

#pragma unroll
        for (int m = 0; m < MB; ++m) {
            acc[m][0] = wave_sum(acc[m][0]);
            acc[m][1] = wave_sum(acc[m][1]);
        }
        if (active) {
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
                        float* o = (a.st ? a.st->logits : a.out) + (size_t)row * a.ldo + n0;
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
        launch_kernel((gemv_kernel<WT, 1, EPI, NORM>), grid, dim3(kThreads), 0, s, a);
    } else if (a.M == 2) {
        launch_kernel((gemv_kernel<WT, 2, EPI, NORM>), grid, dim3(kThreads), 0, s, a);
    } else {
        launch_kernel((gemv_kernel<WT, 4, EPI, NORM>), grid, dim3(kThreads), 0, s, a);
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

hipError_t launch_gemv(int wtype, int epi, const GemvArgs& a, hipStream_t s) {
    switch (wtype) {
        case kStoreF32: return launch_typed<float>(epi, a, s);
        case kStoreBf16: return launch_typed<bf16>(epi, a, s);
        case kStoreF16: return launch_typed<f16>(epi, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace llk
