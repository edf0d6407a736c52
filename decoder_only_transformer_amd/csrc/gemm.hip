// bf16 MFMA GEMM for the prefill projections (gfx950 v_mfma_f32_16x16x32_bf16).
//
// C[m][n] = sum_k A[m][k] * W[n][k], A = bf16 activations [M][lda], W = nn.Linear weight
// [N][K] bf16 (row-major, so both operands are K-contiguous and load as 16-byte chunks).
// 256 threads = 2x2 waves; a workgroup owns a BM x BN tile, each wave (BM/2) x (BN/2) as a
// grid of 16x16 MFMA accumulators.  K advances 64 at a time through double-buffered LDS
// tiles (rows padded by 16 bytes so the 16-lane fragment reads hit distinct banks); the
// next tile's global loads are issued before the current tile's MFMAs.
// Epilogues: RoPE + q store + KV-cache append ([wq; wk; wv]), residual add (wo, w2),
// SiLU gate (w1 and w3 interleaved in one B tile so each wave holds matching gate/up
// accumulators), fp32 store (logits).
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;
constexpr int LDK = BK + 8;   // padded LDS row (elements)

template <int BN, int EPI>
__device__ __forceinline__ const uint16_t* b_row_ptr(const GemmArgs& a, int tile_n, int brow, bool& ok) {
    int n;
    const uint16_t* mat;
    if (EPI == EPI_SWIGLU) {
        constexpr int half = BN / 4;
        const int wn = brow / (BN / 2), jj = brow % (BN / 2);
        n = tile_n * (BN / 2) + wn * half + (jj % half);
        mat = static_cast<const uint16_t*>(jj < half ? a.w0 : a.w1);
    } else if (EPI == EPI_QKV) {
        n = tile_n * BN + brow;
        ok = n < a.N;
        const int nn = ok ? n : 0;
        const int nq = a.qkv.nq, nk = a.qkv.nk;
        if (nn < nq) return static_cast<const uint16_t*>(a.w0) + (size_t)nn * a.K;
        if (nn < nq + nk) return static_cast<const uint16_t*>(a.w1) + (size_t)(nn - nq) * a.K;
        return static_cast<const uint16_t*>(a.w2) + (size_t)(nn - nq - nk) * a.K;
    } else {
        n = tile_n * BN + brow;
        mat = static_cast<const uint16_t*>(a.w0);
    }
    ok = n < a.N;
    return mat + (size_t)(ok ? n : 0) * a.K;
}

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int A_LD = BM * 8 / 256, B_LD = BN * 8 / 256;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][LDK];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int tile_n = blockIdx.x, tile_m = blockIdx.y;
    const int m0 = tile_m * BM;

    const uint16_t* ap[A_LD];
    bool aok[A_LD];
    int arow[A_LD], acol[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int c = tid + 256 * i;
        arow[i] = c >> 3;
        acol[i] = (c & 7) * 8;
        const int gm = m0 + arow[i];
        aok[i] = gm < a.M;
        ap[i] = static_cast<const uint16_t*>(a.a) + (size_t)(aok[i] ? gm : 0) * a.lda + acol[i];
    }
    const uint16_t* bp[B_LD];
    bool bok[B_LD];
    int brow[B_LD], bcol[B_LD];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int c = tid + 256 * i;
        brow[i] = c >> 3;
        bcol[i] = (c & 7) * 8;
        bool ok = true;
        bp[i] = b_row_ptr<BN, EPI>(a, tile_n, brow[i], ok) + bcol[i];
        bok[i] = ok;
    }

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 ra[A_LD], rb[B_LD];
    const uint4 zero = make_uint4(0, 0, 0, 0);
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) ra[i] = aok[i] ? ld16(ap[i] + (size_t)kt * BK) : zero;
#pragma unroll
        for (int i = 0; i < B_LD; ++i) rb[i] = bok[i] ? ld16_stream(bp[i] + (size_t)kt * BK) : zero;
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) *reinterpret_cast<uint4*>(&As[buf][arow[i]][acol[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_LD; ++i) *reinterpret_cast<uint4*>(&Bs[buf][brow[i]][bcol[i]]) = rb[i];
    };

    const int nk = a.K / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    const int fr = lane & 15, fk = (lane >> 4) * 8;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            bf16x8_t af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const bf16x8_t*>(&As[buf][wm * WM + i * 16 + fr][ks + fk]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[buf][wn * WN + j * 16 + fr][ks + fk]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // Epilogue.  Lane holds C[row0 + e][col] for e = 0..3 of each 16x16 tile.
    const int rq = (lane >> 4) * 4;
    if (EPI == EPI_SWIGLU) {
        constexpr int half = BN / 4;
        uint16_t* out = static_cast<uint16_t*>(a.out16);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN / 2; ++j) {
                const int unit = tile_n * (BN / 2) + wn * half + j * 16 + fr;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = m0 + wm * WM + i * 16 + rq + e;
                    if (m < a.M && unit < a.N)
                        out[(size_t)m * a.ldo16 + unit] = f32_to_bf16(silu(acc[i][j][e]) * acc[i][j + TN / 2][e]);
                }
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = tile_n * BN + wn * WN + j * 16 + fr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * WM + i * 16 + rq + e;
                float v = acc[i][j][e];
                if (EPI == EPI_QKV) {
                    const float partner = __shfl_xor(v, 1, kWave);
                    if (m >= a.M || n >= a.N) continue;
                    const QkvTarget& t = a.qkv;
                    const int b = m / t.seqlen;
                    const int pos = t.start_pos + (m - b * t.seqlen);
                    if (n < t.nq + t.nk) {
                        const float2 cs = t.rope[(size_t)pos * (t.head_dim / 2) + (n % t.head_dim) / 2];
                        v = (n & 1) ? partner * cs.y + v * cs.x : v * cs.x - partner * cs.y;
                    }
                    if (n < t.nq) {
                        t.q[(size_t)m * t.nq + n] = v;
                    } else {
                        const bool is_k = n < t.nq + t.nk;
                        const int c = is_k ? n - t.nq : n - t.nq - t.nk;
                        uint16_t* cache = static_cast<uint16_t*>(is_k ? t.cache_k : t.cache_v);
                        cache[((size_t)b * t.max_seq + pos) * (size_t)t.nk + c] = f32_to_bf16(v);
                    }
                } else if (m < a.M && n < a.N) {
                    if (EPI == EPI_RESID)
                        a.resid[(size_t)m * a.ldr + n] += v;
                    else
                        a.out[(size_t)m * a.ldo + n] = v;
                }
            }
        }
}

template <int BM, int BN, int EPI>
hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
    const int ncols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const dim3 grid((a.N + ncols - 1) / ncols, (a.M + BM - 1) / BM);
    hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs& a, hipStream_t s) {
    // Small M (short prefill): narrower tiles so enough workgroups stream the weights.
    if (a.M <= 64) return launch_tile<64, 64, EPI>(a, s);
    if (a.M <= 256) return launch_tile<128, 64, EPI>(a, s);
    return launch_tile<128, 128, EPI>(a, s);
}

}  // namespace

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s) {
    switch (epi) {
        case EPI_QKV: return launch_epi<EPI_QKV>(a, s);
        case EPI_RESID: return launch_epi<EPI_RESID>(a, s);
        case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(a, s);
        default: return launch_epi<EPI_STORE>(a, s);
    }
}

}  // namespace llk
