// Weight-streaming products for a few activation rows on 16-bit MFMA (decode with batch > 4;
// bf16 or fp16, the storage type T16 of the weights and the 16-bit activations).
//
// y[m][n] = sum_k x[m][k] * W[n][k] for M <= 32 rows.  The vector-ALU GEMV would spend M FMAs
// per weight element; here the weights are the MFMA A operand (16 output rows) and the
// activations the B operand (batch rows as MFMA columns).
//
// Memory access is what matters.  A 16-row A fragment loaded straight from a row-major
// matrix touches 16 rows per quarter-wave and ran at half of HBM bandwidth, so:
//  - weights go global -> LDS with global_load_lds_dwordx4, 8 rows x 128 bytes per wave
//    instruction (lanes 8r..8r+7 read the chunks of row r: whole cache lines); lane 8r + s
//    fetches chunk s ^ r, so that a fragment read (16 rows, one chunk each) hits distinct
//    LDS banks;
//  - activations arrive in fragment-major order (their producer wrote them that way; see
//    frag_index), so a wave's B fragment is one contiguous 1 KB load.
// A workgroup owns NT blocks of 16 output rows; its waves take interleaved stages of 64 k
// (128 bytes of each row), each wave through a ring of its own (D slots, D - 1 stages in
// flight), with no barrier inside the loop.  Every activation fragment a wave loads feeds
// the MFMAs of all NT (x NW matrices) weight blocks: with 32 batch rows the activations are
// as many bytes per stage as one weight block, and the bytes a CU takes in per stage, not
// the weights alone, set the pace.  At the end the waves' partial sums meet in LDS.
// Epilogues: RoPE + 16-bit q / KV append, residual add, SiLU gate (16-bit out, optionally in
// fragment-major order for the next product), fp32 logits.  A residual product may split K
// over gridDim.y (SkinnyArgs::ksplit): each split then stores its fp32 sum, and the RMSNorm
// launched next adds the splits to the residual in split order.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr int kSkBK = 64;          // k per stage: 128 bytes of every row
constexpr int kSkWBytes = 2048;    // one matrix's stage for one wave: 16 rows x 128 bytes

template <typename T16>
__device__ __forceinline__ typename Mma<T16>::v8 frag(const uint4& v) {
    return __builtin_bit_cast(typename Mma<T16>::v8, u32x4_t{v.x, v.y, v.z, v.w});
}
template <typename T16>
__device__ __forceinline__ typename Mma<T16>::v8 frag(const u32x4_t& v) {
    return __builtin_bit_cast(typename Mma<T16>::v8, v);
}

// Byte offset, inside a block of 8 rows x 128 bytes, of 16-byte chunk c of row r.
__device__ __forceinline__ int sk_slot(int r, int c) { return (8 * r + (c ^ r)) * 16; }

// Two LDS fragment reads that wait for their own results (the compiler then has no LDS read
// to order after the ring's DMA writes, which it cannot tell apart from this stage's).
__device__ __forceinline__ void lds_read2(u32x4_t& r0, u32x4_t& r1, uint32_t a0, uint32_t a1) {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1)
        : "v"(a0), "v"(a1)
        : "memory");
}

// Pointer to row n of the weight matrix `w` of the product (QKV: the row of wq, wk or wv).
template <int EPI>
__device__ __forceinline__ const uint16_t* sk_row(const SkinnyArgs& a, int w, int n) {
    if (EPI == EPI_QKV) {
        const int nq = a.qkv.nq, nk = a.qkv.nk;
        const void* m = n < nq ? a.w0 : (n < nq + nk ? a.w1 : a.w2);
        const int r = n < nq ? n : (n < nq + nk ? n - nq : n - nq - nk);
        return static_cast<const uint16_t*>(m) + (size_t)r * a.K;
    }
    return static_cast<const uint16_t*>(w == 0 ? a.w0 : a.w1) + (size_t)n * a.K;
}

// Epilogue of one 16 x 16 result tile: acc[w][e] = y[m][n = nb + 4g + e] of matrix w.
template <typename T16, int NW, int EPI>
__device__ __forceinline__ void sk_epilogue(const SkinnyArgs& a, const f32x4 (&acc)[NW], int m, int nb, int g) {
    if (m >= a.M) return;
    if (EPI == EPI_QKV) {
        const QkvTarget& q = a.qkv;
        const int b = m / q.seqlen;
        const int pos = (q.st ? q.st->pos : q.start_pos) + (m - b * q.seqlen);
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
            const int n = nb + 4 * g + e;
            if (n >= a.N) continue;
            float y0 = acc[0][e], y1 = acc[0][e + 1];
            if (n < q.nq + q.nk) {
                const float2 cs = q.rope[(size_t)pos * (q.head_dim / 2) + (n % q.head_dim) / 2];
                const float r0 = y0 * cs.x - y1 * cs.y;
                const float r1 = y0 * cs.y + y1 * cs.x;
                y0 = r0;
                y1 = r1;
            }
            if (n < q.nq) {
                q.q[(size_t)m * q.nq + n] = Mma<T16>::round(y0);
                q.q[(size_t)m * q.nq + n + 1] = Mma<T16>::round(y1);
            } else {
                const bool is_k = n < q.nq + q.nk;
                const int c = is_k ? n - q.nq : n - q.nq - q.nk;
                uint16_t* cache = static_cast<uint16_t*>(is_k ? q.cache_k : q.cache_v);
                *reinterpret_cast<uint32_t*>(cache + ((size_t)b * q.max_seq + pos) * (size_t)q.nk + c) =
                    Mma<T16>::pack2(y0, y1);
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int n = nb + 4 * g + e;
            if (n >= a.N) continue;
            if (EPI == EPI_RESID) {
                if (a.ksplit > 1)   // this K split's share, summed into the residual later
                    a.part[((size_t)blockIdx.y * a.M + m) * a.N + n] = acc[0][e];
                else
                    a.resid[(size_t)m * a.ldr + n] += acc[0][e];
            } else if (EPI == EPI_SWIGLU) {
                const size_t o = a.out_frag_mt ? frag_index(m, n, a.out_frag_mt) : (size_t)m * a.ldo + n;
                static_cast<uint16_t*>(a.out16)[o] = Mma<T16>::bits(silu(acc[0][e]) * acc[NW - 1][e]);
            } else {
                (a.st ? a.st->logits : a.out)[(size_t)m * a.ldo + n] = acc[0][e];
            }
        }
    }
}

template <typename T16, int NW, int NT, int MT, int EPI, int D, int NWV>
__global__ __launch_bounds__(64 * NWV) void skinny_kernel(SkinnyArgs a) {
    constexpr int NB = NT * NW;                   // weight blocks (16 rows each) per stage
    constexpr int kStage = NB * kSkWBytes;        // one wave's ring slot
    constexpr int kOps = 2 * NB + 2 * MT;         // loads per wave per stage (DMA + fragments)
    constexpr int kWait = (D - 2) * kOps;         // loads of later stages left in flight
    static_assert(kWait < 64, "vmcnt holds at most 63");
    static_assert(NWV * D * kStage >= NWV * NB * MT * 64 * 16, "the reduction reuses the ring");
    static_assert(NT * MT <= NWV, "one wave per result tile in the epilogue");
    __shared__ __attribute__((aligned(1024))) uint8_t ring[NWV * D * kStage];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int fr = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16 * NT;
    // K split blockIdx.y of gridDim.y takes stages st0 .. st0 + nst - 1
    const int nst_all = a.K / kSkBK;
    const int st0 = (int)((int64_t)blockIdx.y * nst_all / gridDim.y);
    const int nst = (int)((int64_t)(blockIdx.y + 1) * nst_all / gridDim.y) - st0;
    const int n_my = (nst - wid + NWV - 1) / NWV;     // stages wid, wid + NWV, ... of this wave

    // DMA sources of this lane: rows n0 + 16t + 8h + r8 (clamped past N), chunk c8
    const int r8 = lane >> 3, c8 = (lane & 7) ^ r8;
    const uint16_t* wsrc[NT][NW][2];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                wsrc[t][w][h] = sk_row<EPI>(a, w, min(n0 + 16 * t + 8 * h + r8, a.N - 1)) + c8 * 8;
    // fragment-major activations: tile t of k-step s is the 1 KB at element (s * MT + t) * 512
    const uint16_t* xsrc = static_cast<const uint16_t*>(a.x) + lane * 8;

    uint8_t* wring = ring + wid * D * kStage;
    const uint32_t wring_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)wring));
    uint4 xr[D][2][MT];     // activation fragments of the stages in flight

    // Workgroups start at rotated points of K: with every workgroup at the same k, the rows'
    // chunks (a fixed stride apart) crowd onto the same HBM channels.
    const int rot = (int)((blockIdx.x * 37u) % (unsigned)nst);
    auto issue = [&](int i, int u) {
        int kt = min(wid + NWV * i, nst - 1) + rot;     // repeats of the last stage past the end
        kt = (kt >= nst ? kt - nst : kt) + st0;
        const int k = kt * kSkBK;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                __builtin_amdgcn_global_load_lds((gbl_void_t*)(wsrc[b / NW][b % NW][h] + k),
                                                 (lds_void_t*)(wring + u * kStage + b * kSkWBytes + h * 1024), 16, 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int t = 0; t < MT; ++t) xr[u][j][t] = ld16(xsrc + (size_t)((2 * kt + j) * MT + t) * 512);
    };

    // A fragment offsets in a slot for the two k-steps of a stage (chunks 4j + g)
    const uint32_t aoff0 = (fr >> 3) * 1024 + sk_slot(fr & 7, g);
    const uint32_t aoff1 = (fr >> 3) * 1024 + sk_slot(fr & 7, 4 + g);

    f32x4 acc[NB][MT];    // block b = weight rows n0 + 16 (b / NW), matrix b % NW
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[b][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // live = 0 (a step past this wave's last stage): the weight fragments are masked to zero,
    // so the product adds nothing; no branch, so the loop body stays straight-line
    auto compute = [&](int u, uint32_t live) {
        const uint32_t sb = wring_addr + u * kStage;
        u32x4_t ra[NB][2];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            lds_read2(ra[b][0], ra[b][1], sb + b * kSkWBytes + aoff0, sb + b * kSkWBytes + aoff1);
            ra[b][0] &= live;
            ra[b][1] &= live;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[b][t] = Mma<T16>::mma(frag<T16>(ra[b][j]), frag<T16>(xr[u][j][t]), acc[b][t]);
    };

#pragma unroll
    for (int u = 0; u < D - 1; ++u) issue(u, u);
    // Whole ring revolutions with a straight-line body: steps past this wave's last stage
    // still wait and issue (repeats) and add zero, so the loop has one path and the
    // compiler's own wait counts stay exact across its back edge.
    for (int i0 = 0; i0 < n_my; i0 += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            // this wave's loads of step i0 + u have landed once only those of the D - 2 later
            // steps are outstanding; its reads of the previous slot finished in compute
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWait) : "memory");
            issue(i0 + u + D - 1, (u + D - 1) % D);
            compute(u, i0 + u < n_my ? 0xffffffffu : 0u);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the repeated tail loads

    // sum the waves' partials: red[wave][b][t][lane] in the ring's memory
    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(ring);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int t = 0; t < MT; ++t) red[((wid * NB + b) * MT + t) * 64 + lane] = acc[b][t];
    __syncthreads();
    // wave q finishes result tile (row block q / MT, batch rows 16 (q % MT) .. + 15)
    if (wid >= NT * MT) return;
    const int tb = wid / MT, tm = wid % MT;
    f32x4 sum[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        sum[w] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < NWV; ++q) sum[w] += red[((q * NB + tb * NW + w) * MT + tm) * 64 + lane];
    }
    sk_epilogue<T16, NW, EPI>(a, sum, 16 * tm + fr, n0 + 16 * tb, g);
}

template <typename T16, int NW, int NT, int MT, int EPI, int D, int NWV>
hipError_t launch_waves(const SkinnyArgs& a, hipStream_t s) {
    const dim3 grid((a.N + 16 * NT - 1) / (16 * NT), EPI == EPI_RESID && a.ksplit > 1 ? a.ksplit : 1);
    launch_kernel((skinny_kernel<T16, NW, NT, MT, EPI, D, NWV>), grid, dim3(64 * NWV), 0, s, a);
    return hipGetLastError();
}

// Row blocks per workgroup (NT), ring depth per wave (D) and waves per workgroup (NWV), from
// timings at the decode shapes (batch 8 .. 32 of the 7B, 13B and 70B layer widths):
//  - SiLU gate: gate and up rows already share each activation fragment: NT = 1, D = 4, and
//    8 waves when there are too few 16-row tiles for two 4-wave workgroups per CU;
//  - wide products (q/k/v, logits: 640 or more tiles): NT = 4 for up to 16 batch rows; for up
//    to 32, NT = 3 with 8 waves and a 2-slot ring at up to 1024 tiles (the 7B q/k/v: one
//    workgroup per CU), else NT = 2 with 4 waves;
//  - the others (wo, w2): NT = 2 with 8 waves for up to 16 rows, NT = 1 with 4 for more;
//  - residual products split over K (fewer than 512 tiles: the 7B wo/w2 at 32 rows and the
//    13B ones at 16 filled half the chip or less): 4 waves, NT = 1 for up to 16 rows, NT = 2
//    for more (7B w2 at 32 rows 27.8 -> 21.6 us, 13B wo at 16 rows 19.5 -> 15.7 us).
// The LDS of a workgroup stays at or under 128 KB.
template <typename T16, int EPI>
hipError_t launch_epi(const SkinnyArgs& a, hipStream_t s) {
    const int tiles = (a.N + 15) / 16;
    const bool m16 = a.M <= 16;     // one 16-row batch tile (MT = 1) or two
    if constexpr (EPI == EPI_RESID) {
        if (a.ksplit > 1) return m16 ? launch_waves<T16, 1, 1, 1, EPI, 4, 4>(a, s) : launch_waves<T16, 1, 2, 2, EPI, 4, 4>(a, s);
    }
    if constexpr (EPI == EPI_SWIGLU) {
        if (tiles >= 512) return m16 ? launch_waves<T16, 2, 1, 1, EPI, 4, 4>(a, s) : launch_waves<T16, 2, 1, 2, EPI, 4, 4>(a, s);
        return m16 ? launch_waves<T16, 2, 1, 1, EPI, 4, 8>(a, s) : launch_waves<T16, 2, 1, 2, EPI, 4, 8>(a, s);
    } else {
        if (tiles >= 640) {
            if (m16) return launch_waves<T16, 1, 4, 1, EPI, 4, 4>(a, s);
            // about one workgroup per CU: 3 row blocks, 8 waves, a 2-slot ring each
            if (tiles <= 1024) return launch_waves<T16, 1, 3, 2, EPI, 2, 8>(a, s);
            return launch_waves<T16, 1, 2, 2, EPI, 4, 4>(a, s);
        }
        return m16 ? launch_waves<T16, 1, 2, 1, EPI, 4, 8>(a, s) : launch_waves<T16, 1, 1, 2, EPI, 6, 4>(a, s);
    }
}

}  // namespace

int skinny_resid_splits(int M, int N, int K) {
    if (M < 1 || M > 32 || K % kSkBK != 0) return 1;
    // two splits while the row blocks alone leave CUs idle, each split at least 8 stages
    return (N + 15) / 16 < 512 && K / kSkBK >= 16 ? 2 : 1;
}

hipError_t launch_skinny(int epi, const SkinnyArgs& a, hipStream_t s) {
    if (a.M < 1 || a.M > 32 || a.K % kSkBK != 0 || a.K < kSkBK) return hipErrorInvalidValue;
    if (a.ksplit > 1 && (epi != EPI_RESID || !a.part || a.ksplit > a.K / kSkBK)) return hipErrorInvalidValue;
    if (a.wtype == kStoreF16) {
        switch (epi) {
            case EPI_QKV: return launch_epi<f16, EPI_QKV>(a, s);
            case EPI_RESID: return launch_epi<f16, EPI_RESID>(a, s);
            case EPI_SWIGLU: return launch_epi<f16, EPI_SWIGLU>(a, s);
            default: return launch_epi<f16, EPI_STORE>(a, s);
        }
    }
    if (a.wtype != kStoreBf16) return hipErrorInvalidValue;
    switch (epi) {
        case EPI_QKV: return launch_epi<bf16, EPI_QKV>(a, s);
        case EPI_RESID: return launch_epi<bf16, EPI_RESID>(a, s);
        case EPI_SWIGLU: return launch_epi<bf16, EPI_SWIGLU>(a, s);
        default: return launch_epi<bf16, EPI_STORE>(a, s);
    }
}

}  // namespace llk
