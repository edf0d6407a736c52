// bf16 MFMA GEMM for the prefill projections (gfx950 v_mfma_f32_16x16x32_bf16).
//
// C[m][n] = sum_k A[m][k] * W[n][k], A = bf16 activations [M][lda], W = nn.Linear weight
// [N][K] bf16 (row-major, so both operands are K-contiguous and load as 16-byte chunks).
// A workgroup of WGM x WGN waves owns a BM x BN tile, each wave (BM/WGM) x (BN/WGN) as a grid
// of 16x16 MFMA accumulators.  K advances 64 at a time through double-buffered LDS tiles
// (rows padded by 16 bytes so the 16-lane fragment reads hit distinct banks); the next
// tile's global loads are issued before the current tile's MFMAs.  Workgroups are mapped to
// tiles XCD-aware: the dispatcher deals workgroup ids round-robin over the 8 XCDs, so each
// XCD is given a contiguous share of the tile space, walked in groups of 8 M-tiles so the
// workgroups resident on one XCD share A and B tiles in its L2.
// Epilogues: RoPE + q store + KV-cache append ([wq; wk; wv]), residual add (wo, w2),
// SiLU gate (w1 and w3 interleaved in one B tile so each wave holds matching gate/up
// accumulators), fp32 store (logits).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 64;
constexpr int LDK = BK + 8;   // padded LDS row (elements)

// Weight row feeding row `brow` of the B tile.  For the SiLU gate each wave column's share
// of the tile is half w1 rows and half the matching w3 rows.
template <int BN, int WGN, int EPI>
__device__ __forceinline__ const uint16_t* b_row_ptr(const GemmArgs& a, int tile_n, int brow, bool& ok) {
    int n;
    const uint16_t* mat;
    if (EPI == EPI_SWIGLU) {
        constexpr int half = BN / WGN / 2;
        const int wn = brow / (BN / WGN), jj = brow % (BN / WGN);
        n = tile_n * (BN / 2) + wn * half + (jj % half);
        mat = static_cast<const uint16_t*>(jj < half ? a.w0 : a.w1);
    } else if (EPI == EPI_QKV || EPI == EPI_STORE_QKV) {
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

constexpr int kXcds = 8;
constexpr int kGroupM = 8;

// Tile (tm, tn) of linear workgroup id `id` (see the header comment).  The grid is padded to
// kXcds * ceil(total / kXcds) workgroups, on which id -> t is a bijection; returns false for
// the few ids whose t falls past the last tile.
__device__ __forceinline__ bool tile_of(int id, int n_tm, int n_tn, int& tm, int& tn) {
    const int total = n_tm * n_tn;
    const int per_xcd = (total + kXcds - 1) / kXcds;
    const int t = (id % kXcds) * per_xcd + id / kXcds;
    if (t >= total) return false;
    const int group = t / (kGroupM * n_tn);
    const int first_m = group * kGroupM;
    const int gsize = min(kGroupM, n_tm - first_m);
    const int r = t - group * kGroupM * n_tn;
    tm = first_m + r % gsize;
    tn = r / gsize;
    return true;
}

// Epilogue.  Lane holds C[row0 + e][col] for e = 0..3 of each 16x16 accumulator tile.
template <int BN, int WGN, int TM, int TN, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& a, f32x4 (&acc)[TM][TN], int m0, int tile_n,
                                         int wm, int wn, int lane) {
    constexpr int WM = TM * 16, WN = TN * 16;
    const int fr = lane & 15;
    const int rq = (lane >> 4) * 4;
    if (EPI == EPI_SWIGLU) {
        constexpr int half = BN / WGN / 2;
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
                        t.q[(size_t)m * t.nq + n] = round_bf16(v);
                    } else {
                        const bool is_k = n < t.nq + t.nk;
                        const int c = is_k ? n - t.nq : n - t.nq - t.nk;
                        uint16_t* cache = static_cast<uint16_t*>(is_k ? t.cache_k : t.cache_v);
                        cache[((size_t)b * t.max_seq + pos) * (size_t)t.nk + c] = f32_to_bf16(v);
                    }
                } else if (m < a.M && n < a.N) {
                    if (EPI == EPI_RESID) {
                        if (gridDim.z > 1)
                            a.part[((size_t)blockIdx.z * a.M + m) * a.N + n] = v;
                        else
                            a.resid[(size_t)m * a.ldr + n] += v;
                    } else {
                        a.out[(size_t)m * a.ldo + n] = v;
                    }
                }
            }
        }
}

template <int BM, int BN, int WGM, int WGN, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(GemmArgs a, int n_tm, int n_tn) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int A_LD = BM * 8 / NT, B_LD = BN * 8 / NT;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][LDK];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WGN, wn = wid % WGN;
    int tile_m, tile_n;
    if (!tile_of(blockIdx.x, n_tm, n_tn, tile_m, tile_n)) return;
    const int m0 = tile_m * BM;
    // K range of this workgroup (split-K over gridDim.z, in BK steps)
    const int nk_all = a.K / BK;
    const int kt0 = (int)((int64_t)nk_all * blockIdx.z / gridDim.z);
    const int kt1 = (int)((int64_t)nk_all * (blockIdx.z + 1) / gridDim.z);

    const uint16_t* ap[A_LD];
    bool aok[A_LD];
    int arow[A_LD], acol[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int c = tid + NT * i;
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
        const int c = tid + NT * i;
        brow[i] = c >> 3;
        bcol[i] = (c & 7) * 8;
        bool ok = true;
        bp[i] = b_row_ptr<BN, WGN, EPI>(a, tile_n, brow[i], ok) + bcol[i];
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

    gload(kt0);
    lstore(0);
    __syncthreads();
    const int fr = lane & 15, fk = (lane >> 4) * 8;
    for (int kt = kt0; kt < kt1; ++kt) {
        const int buf = (kt - kt0) & 1;
        if (kt + 1 < kt1) gload(kt + 1);
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
        if (kt + 1 < kt1) lstore(buf ^ 1);
        __syncthreads();
    }

    epilogue<BN, WGN, TM, TN, EPI>(a, acc, m0, tile_n, wm, wn, lane);
}

// resid[m][n] += sum over splits of part[z][m][n], in split order.
__global__ void splitk_reduce_kernel(const float* part, int splits, int M, int N, float* resid,
                                     int64_t ldr) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)M * N) return;
    const int m = (int)(i / N), n = (int)(i - (size_t)m * N);
    float v = 0.f;
    for (int z = 0; z < splits; ++z) v += part[(size_t)z * M * N + i];
    resid[(size_t)m * ldr + n] += v;
}

template <int BM, int BN, int WGM, int WGN, int EPI>
hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
    const int ncols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int splits = (EPI == EPI_RESID && a.part) ? std::max(1, a.splits) : 1;
    const int n_tn = (a.N + ncols - 1) / ncols, n_tm = (a.M + BM - 1) / BM;
    const int per_xcd = (n_tn * n_tm + kXcds - 1) / kXcds;
    const dim3 grid(per_xcd * kXcds, 1, splits);
    launch_kernel((gemm_kernel<BM, BN, WGM, WGN, EPI>), grid, dim3(64 * WGM * WGN), 0, s, a, n_tm, n_tn);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const size_t n = (size_t)a.M * a.N;
    launch_kernel(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       a.part, splits, a.M, a.N, a.resid, a.ldr);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------------------
// Large-M variant: 256x256 tiles, 8 waves (4 x 2, 64 x 128 each), K in stages of 32 through
// a 4-deep LDS ring filled by global_load_lds_dwordx4 (global -> LDS without registers),
// loads issued 3 stages ahead.  A wave's load instruction fills 1 KB of LDS contiguously
// (lane i -> bytes 16i..16i+15), i.e. 16 rows x 4 chunks of a 64-byte row; each lane fetches
// the global chunk (chunk ^ swz(row)), so a fragment read of (row, chunk) finds it at slot
// chunk ^ swz(row) and the 16 rows of a fragment land on distinct banks without padding.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr int kBigBM = 256, kBigBN = 256, kBigBK = 32, kBigStages = 4;

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

// One LDS ring slot: a distinct object per stage, so the compiler can tell a fragment read
// of one stage from the DMA writes into another and keeps the later stages in flight.
#define LLK_BIG_SLOT(n)                                                                 \
    __shared__ __attribute__((aligned(1024))) uint16_t As##n[kBigBM * kBigBK];         \
    __shared__ __attribute__((aligned(1024))) uint16_t Bs##n[kBigBN * kBigBK];

template <int EPI>
__global__ __launch_bounds__(512) void gemm_big_kernel(GemmArgs a, int n_tm, int n_tn) {
    constexpr int BM = kBigBM, BN = kBigBN, BKS = kBigBK;
    constexpr int WGN = 2, TM = 4, TN = 8, WM = 64, WN = 128;
    static_assert(kBigStages == 4, "the ring below has four slots");
    LLK_BIG_SLOT(0)
    LLK_BIG_SLOT(1)
    LLK_BIG_SLOT(2)
    LLK_BIG_SLOT(3)
    uint16_t* const Aslot[4] = {As0, As1, As2, As3};
    uint16_t* const Bslot[4] = {Bs0, Bs1, Bs2, Bs3};

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WGN, wn = wid % WGN;
    int tile_m, tile_n;
    if (!tile_of(blockIdx.x, n_tm, n_tn, tile_m, tile_n)) return;
    const int m0 = tile_m * BM;

    // This lane's two A rows and two B rows (one per load instruction of the wave).
    const uint16_t* ap[2];
    const uint16_t* bp[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = (2 * wid + i) * 16 + (lane >> 2);
        const int gc = (lane & 3) ^ swz(row);
        const int gm = min(m0 + row, a.M - 1);
        ap[i] = static_cast<const uint16_t*>(a.a) + (size_t)gm * a.lda + gc * 8;
        bool ok = true;
        bp[i] = b_row_ptr<BN, WGN, EPI>(a, tile_n, row, ok) + gc * 8;
    }
    const int nk_all = a.K / BKS;
    const int kt0 = (int)((int64_t)nk_all * blockIdx.z / gridDim.z);
    const int kt1 = (int)((int64_t)nk_all * (blockIdx.z + 1) / gridDim.z);

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int fr = lane & 15, g = lane >> 4;
    int a_off[TM], b_off[TN];      // element offsets of this lane's fragments in a slot
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = wm * WM + i * 16 + fr;
        a_off[i] = row * BKS + ((g ^ swz(row)) * 8);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int row = wn * WN + j * 16 + fr;
        b_off[j] = row * BKS + ((g ^ swz(row)) * 8);
    }

    auto issue = [&](int kt, uint16_t* Ad, uint16_t* Bd) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            __builtin_amdgcn_global_load_lds((gbl_void_t*)(ap[i] + (size_t)kt * BKS),
                                             (lds_void_t*)(Ad + (2 * wid + i) * 16 * BKS), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((gbl_void_t*)(bp[i] + (size_t)kt * BKS),
                                             (lds_void_t*)(Bd + (2 * wid + i) * 16 * BKS), 16, 0, 0);
        }
    };
    auto compute = [&](const uint16_t* As_, const uint16_t* Bs_) {
        // Fragment reads go out in asm blocks that wait for their own results: the compiler
        // then sees no LDS read it would have to order after the ring's DMA writes (it cannot
        // tell the slots apart across the loop and would drain every load).  Four groups,
        // each followed by the MFMAs it feeds, so a group's reads overlap the MFMAs before it.
        const uint32_t ab = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)As_));
        const uint32_t bb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)Bs_));
        u32x4_t ra[TM], rb[TN];
        asm volatile(
            "ds_read_b128 %0, %6\n\t"
            "ds_read_b128 %1, %7\n\t"
            "ds_read_b128 %2, %8\n\t"
            "ds_read_b128 %3, %9\n\t"
            "ds_read_b128 %4, %10\n\t"
            "ds_read_b128 %5, %11\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(ra[0]), "=&v"(ra[1]), "=&v"(ra[2]), "=&v"(ra[3]), "=&v"(rb[0]), "=&v"(rb[1])
            : "v"(ab + 2 * a_off[0]), "v"(ab + 2 * a_off[1]), "v"(ab + 2 * a_off[2]),
              "v"(ab + 2 * a_off[3]), "v"(bb + 2 * b_off[0]), "v"(bb + 2 * b_off[1])
            : "memory");
        bf16x8_t af[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = __builtin_bit_cast(bf16x8_t, ra[i]);
#pragma unroll
        for (int jg = 0; jg < TN / 2; ++jg) {
            if (jg > 0) {
                asm volatile(
                    "ds_read_b128 %0, %2\n\t"
                    "ds_read_b128 %1, %3\n\t"
                    "s_waitcnt lgkmcnt(0)"
                    : "=&v"(rb[2 * jg]), "=&v"(rb[2 * jg + 1])
                    : "v"(bb + 2 * b_off[2 * jg]), "v"(bb + 2 * b_off[2 * jg + 1])
                    : "memory");
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, rb[2 * jg + jj]);
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    acc[i][2 * jg + jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf, acc[i][2 * jg + jj], 0, 0, 0);
            }
        }
    };

    // Prologue: stages 0..2 (past the end: duplicates of the last stage, so every step has
    // the same number of loads outstanding).
    issue(min(kt0 + 0, kt1 - 1), As0, Bs0);
    issue(min(kt0 + 1, kt1 - 1), As1, Bs1);
    issue(min(kt0 + 2, kt1 - 1), As2, Bs2);

    // Step for stage kt held in slot S: wait for this wave's loads of that stage (the 8
    // loads of the two later stages may stay in flight) and for its LDS reads of the
    // previous slot, barrier (now every wave's are done), refill the previous slot with
    // stage kt+3, compute.
#define LLK_BIG_STEP(S, PREV)                                                     \
    if (kt + S < kt1) {                                                           \
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");  \
        issue(min(kt + S + 3, kt1 - 1), As##PREV, Bs##PREV);                      \
        compute(As##S, Bs##S);                                                    \
    }
    for (int kt = kt0; kt < kt1; kt += 4) {
        LLK_BIG_STEP(0, 3)
        LLK_BIG_STEP(1, 0)
        LLK_BIG_STEP(2, 1)
        LLK_BIG_STEP(3, 2)
    }
#undef LLK_BIG_STEP
    (void)Aslot;
    (void)Bslot;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain the duplicate tail loads
    epilogue<BN, WGN, TM, TN, EPI>(a, acc, m0, tile_n, wm, wn, lane);
}
#undef LLK_BIG_SLOT

template <int EPI>
hipError_t launch_big(const GemmArgs& a, hipStream_t s) {
    const int ncols = (EPI == EPI_SWIGLU) ? kBigBN / 2 : kBigBN;
    const int splits = (EPI == EPI_RESID && a.part) ? std::max(1, a.splits) : 1;
    const int n_tn = (a.N + ncols - 1) / ncols, n_tm = (a.M + kBigBM - 1) / kBigBM;
    const int per_xcd = (n_tn * n_tm + kXcds - 1) / kXcds;
    launch_kernel((gemm_big_kernel<EPI>), dim3(per_xcd * kXcds, 1, splits), dim3(512), 0, s, a,
                       n_tm, n_tn);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const size_t n = (size_t)a.M * a.N;
    launch_kernel(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       a.part, splits, a.M, a.N, a.resid, a.ldr);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs& a, hipStream_t s) {
    // Small M (short prefill): narrower tiles so enough workgroups stream the weights.
    if (a.M <= 64) return launch_tile<64, 64, 2, 2, EPI>(a, s);
    if (a.M <= 256) return launch_tile<128, 64, 2, 2, EPI>(a, s);
    // (the RoPE/KV-append epilogue does not fit 256x256 tiles without spilling)
    if constexpr (EPI == EPI_QKV) {
        return launch_tile<128, 128, 2, 2, EPI>(a, s);
    } else {
        if (a.M <= 2048) return launch_tile<128, 128, 2, 2, EPI>(a, s);
        return launch_big<EPI>(a, s);
    }
}

}  // namespace

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s) {
    switch (epi) {
        case EPI_QKV: return launch_epi<EPI_QKV>(a, s);
        case EPI_RESID: return launch_epi<EPI_RESID>(a, s);
        case EPI_SWIGLU: return launch_epi<EPI_SWIGLU>(a, s);
        case EPI_STORE_QKV: return launch_epi<EPI_STORE_QKV>(a, s);
        default: return launch_epi<EPI_STORE>(a, s);
    }
}

}  // namespace llk
