// 16-bit MFMA GEMM for the prefill projections (gfx950 v_mfma_f32_16x16x32_bf16 for bf16
// models, v_mfma_f32_16x16x32_f16 for fp16 ones; every kernel takes the storage type T16).
//
// C[m][n] = sum_k A[m][k] * W[n][k], A = 16-bit activations [M][lda], W = nn.Linear weight
// [N][K] of the same type (row-major, so both operands are K-contiguous and load as 16-byte
// chunks).
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
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

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

constexpr int kXcds = 8;
constexpr int kCUs = 256;      // compute units of the device (one 256 x 256 tile each at a time)
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
template <typename T16, int BN, int WGN, int TM, int TN, int EPI>
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
                        out[(size_t)m * a.ldo16 + unit] = Mma<T16>::bits(silu(acc[i][j][e]) * acc[i][j + TN / 2][e]);
                }
            }
        return;
    }
    if (EPI == EPI_QKV) {
        // Rotate q/k pairs (neighbouring columns, one lane apart) with the position's
        // cos/sin, then store q and append k, v to the cache rows of (sequence, position).
        // Column and row terms are computed once per fragment column and row.
        const QkvTarget& t = a.qkv;
        const int hd2 = t.head_dim / 2;
        int ncol[TN], rofs[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            ncol[j] = tile_n * BN + wn * WN + j * 16 + fr;
            rofs[j] = (ncol[j] % t.head_dim) / 2;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm * WM + i * 16 + rq + e;
                const int mm = t.row0 + m;    // row of the bsz x seqlen rectangle
                const int b = mm / t.seqlen;
                const int pos = t.start_pos + (mm - b * t.seqlen);
                const float2* rope_row = t.rope + (size_t)pos * hd2;
                const size_t cache_row = ((size_t)b * t.max_seq + pos) * (size_t)t.nk;
                const bool row_ok = m < a.M;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int n = ncol[j];
                    float v = acc[i][j][e];
                    const float partner = __shfl_xor(v, 1, kWave);
                    if (!row_ok || n >= a.N) continue;
                    if (n < t.nq + t.nk) {
                        const float2 cs = rope_row[rofs[j]];
                        v = (n & 1) ? partner * cs.y + v * cs.x : v * cs.x - partner * cs.y;
                    }
                    if (n < t.nq) {
                        t.q[(size_t)mm * t.nq + n] = Mma<T16>::round(v);
                    } else {
                        const bool is_k = n < t.nq + t.nk;
                        const int c = is_k ? n - t.nq : n - t.nq - t.nk;
                        uint16_t* cache = static_cast<uint16_t*>(is_k ? t.cache_k : t.cache_v);
                        cache[cache_row + c] = Mma<T16>::bits(v);
                    }
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
                const float v = acc[i][j][e];
                if (m < a.M && n < a.N) {
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

template <typename T16, int BM, int BN, int WGM, int WGN, int EPI>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_kernel(GemmArgs a, int n_tm, int n_tn) {
    typedef typename Mma<T16>::v8 v8_t;
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
            v8_t af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const v8_t*>(&As[buf][wm * WM + i * 16 + fr][ks + fk]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bfr[j] = *reinterpret_cast<const v8_t*>(&Bs[buf][wn * WN + j * 16 + fr][ks + fk]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = Mma<T16>::mma(af[i], bfr[j], acc[i][j]);
        }
        if (kt + 1 < kt1) lstore(buf ^ 1);
        __syncthreads();
    }

    epilogue<T16, BN, WGN, TM, TN, EPI>(a, acc, m0, tile_n, wm, wn, lane);
}

// resid[m][n] += sum over splits of part[z][m][n] (rows ldp apart), in split order.
__global__ void splitk_reduce_kernel(const float* part, int splits, int M, int N, int64_t ldp,
                                     float* resid, int64_t ldr) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)M * N) return;
    const int m = (int)(i / N), n = (int)(i - (size_t)m * N);
    float v = 0.f;
    for (int z = 0; z < splits; ++z) v += part[((size_t)z * M + m) * ldp + n];
    resid[(size_t)m * ldr + n] += v;
}

// SiLU gate from split partials of the [w1; w3] product: unit u of row m has its gate in
// B row p and its up projection in B row p + half, where (tile, wave column, offset) of u
// give p (the interleaving the MFMA kernels load w1 and w3 rows in).
template <typename T16>
__global__ void swiglu_reduce_kernel(const float* part, int splits, int M, int N, int64_t ldp,
                                     int bn, int wn_cols, uint16_t* out, int64_t ldo) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)M * N) return;
    const int m = (int)(i / N), u = (int)(i - (size_t)m * N);
    const int half = wn_cols / 2;
    const int tile = u / (bn / 2), r = u % (bn / 2);
    const int p = tile * bn + (r / half) * wn_cols + r % half;
    float g = 0.f, v = 0.f;
    for (int z = 0; z < splits; ++z) {
        const float* row = part + ((size_t)z * M + m) * ldp;
        g += row[p];
        v += row[p + half];
    }
    out[(size_t)m * ldo + u] = Mma<T16>::bits(silu(g) * v);
}

template <typename T16, int BM, int BN, int WGM, int WGN, int EPI>
hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
    const int ncols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int splits = (EPI == EPI_RESID && a.part) ? std::max(1, a.splits) : 1;
    const int n_tn = (a.N + ncols - 1) / ncols, n_tm = (a.M + BM - 1) / BM;
    const int per_xcd = (n_tn * n_tm + kXcds - 1) / kXcds;
    const dim3 grid(per_xcd * kXcds, 1, splits);
    if (a.deferred) *a.deferred = 0;
    launch_kernel((gemm_kernel<T16, BM, BN, WGM, WGN, EPI>), grid, dim3(64 * WGM * WGN), 0, s, a, n_tm, n_tn);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    if (a.deferred && splits <= kMaxNormFold) {   // partials [splits][M][N], folded by the next norm
        *a.deferred = splits;
        return hipSuccess;
    }
    const size_t n = (size_t)a.M * a.N;
    launch_kernel(splitk_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                  a.part, splits, a.M, a.N, (int64_t)a.N, a.resid, a.ldr);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------------------
// LDS-ring kernel of the 128 x 128 tile (short prefills): 8 waves as 2 x 4 of 64 x 32, K in
// stages of 64 through a 3-slot LDS ring filled by global_load_lds_dwordx4 (global -> LDS
// without registers), loads issued NS - 1 stages ahead.  The 256-row tile (gemm_pp_kernel
// below) fills its rings the same way.  Short prefills (a few hundred rows,
// where the weights are the traffic) split K over gridDim.z so enough workgroups stream the
// weights: each split stores its raw fp32 tile [z][M][B row] and a reduce pass applies the
// epilogue (or the next RMSNorm folds the residual products' partials).  A wave's load
// instruction fills 1 KB of LDS contiguously (lane i -> bytes 16i..16i+15), i.e. 8 whole
// 128-byte rows: rows of half a cache line would cost twice the L2 requests for the same
// bytes, and the request rate is what bounds these loads.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr int kBigBN = 256;

// LDS rows are 128 bytes (64 K elements).  The LDS serves a 16-byte read 8 lanes at a time;
// the 8 lanes of a fragment read take 8 consecutive rows at one logical chunk, and storing
// chunk c of row r at slot c ^ (r % 8) puts them on 8 distinct 16-byte slots of the banks
// (without it all 8 would share one).  The load instructions write 1 KB contiguously, so
// each lane fetches the global chunk that belongs at its LDS slot.

// Epilogue of the 256 x 256 kernel through LDS.  A wave's accumulators (64 rows x 128
// columns, 4 consecutive rows of one column per lane and tile) go to its own 16 KB of the
// then idle ring as fp32, 64 columns per pass, and come back as 16-byte row chunks, 16 lanes
// to a row: the residual rows are read and written, and the q / K / V / gated rows written,
// in whole 256-byte segments rather than 4-byte pieces.  Chunks (4 floats) are XOR-swizzled
// by row so that both the column-wise writes and the row-wise reads spread over the banks.
// RoPE is applied on the row chunks: a lane holds two whole (even, odd) pairs.
template <typename T16, int EPI>
__device__ __forceinline__ void epilogue_staged(const GemmArgs& a, f32x4 (&acc)[4][8], int m0, int tile_n,
                                                int wm, int wn, int lane, float* stage) {
    constexpr int TM = 4, WM = 64, WN = 128;
    const int fr = lane & 15, rq = (lane >> 4) * 4;
    const int row0 = m0 + wm * WM;
    auto phys = [](int r, int chunk) { return r * 64 + ((chunk ^ (4 * ((r >> 2) & 3))) << 2); };
    constexpr int kPasses = (EPI == EPI_SWIGLU) ? 1 : 2;
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
        __syncthreads();    // the ring's last reads (or the previous pass's) are done
        // phase 1: the 4 column tiles of this pass, fp32
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = i * 16 + rq + e, col = jj * 16 + fr;
                    float v;
                    if constexpr (EPI == EPI_SWIGLU)
                        v = silu(acc[i][jj][e]) * acc[i][jj + 4][e];
                    else
                        v = acc[i][pass * 4 + jj][e];
                    stage[phys(r, col >> 2) + (col & 3)] = v;
                }
        __syncthreads();
        // phase 2: row chunks, 4 rows per step
#pragma unroll 4
        for (int it = 0; it < 16; ++it) {
            const int r = it * 4 + (lane >> 4), c = lane & 15;
            const int m = row0 + r;
            if (m >= a.M) continue;
            const float4 v = *reinterpret_cast<const float4*>(stage + phys(r, c));
            if constexpr (EPI == EPI_RESID) {
                const int n = tile_n * 256 + wn * WN + pass * 64 + c * 4;
                if (n >= a.N) continue;
                float4* dst = reinterpret_cast<float4*>(a.resid + (size_t)m * a.ldr + n);
                float4 h = *dst;
                h.x += v.x;
                h.y += v.y;
                h.z += v.z;
                h.w += v.w;
                *dst = h;
            } else if constexpr (EPI == EPI_SWIGLU) {
                const int n = tile_n * 128 + wn * 64 + c * 4;
                if (n >= a.N) continue;
                uint2 p;
                p.x = Mma<T16>::pack2(v.x, v.y);
                p.y = Mma<T16>::pack2(v.z, v.w);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out16) + (size_t)m * a.ldo16 + n) = p;
            } else {
                const QkvTarget& t = a.qkv;
                const int n = tile_n * 256 + wn * WN + pass * 64 + c * 4;
                if (n >= a.N) continue;
                const int mm = t.row0 + m;    // row of the bsz x seqlen rectangle
                const int b = mm / t.seqlen;
                const int pos = t.start_pos + (mm - b * t.seqlen);
                float4 y = v;
                if (n < t.nq + t.nk) {
                    // (cos, sin) of the pairs (n, n + 1) and (n + 2, n + 3)
                    const float4 cs = *reinterpret_cast<const float4*>(
                        t.rope + (size_t)pos * (t.head_dim / 2) + (n % t.head_dim) / 2);
                    y.x = v.x * cs.x - v.y * cs.y;
                    y.y = v.y * cs.x + v.x * cs.y;
                    y.z = v.z * cs.z - v.w * cs.w;
                    y.w = v.w * cs.z + v.z * cs.w;
                }
                if (n < t.nq) {
                    *reinterpret_cast<float4*>(t.q + (size_t)mm * t.nq + n) =
                        float4{Mma<T16>::round(y.x), Mma<T16>::round(y.y), Mma<T16>::round(y.z), Mma<T16>::round(y.w)};
                } else {
                    const bool is_k = n < t.nq + t.nk;
                    const int cc = is_k ? n - t.nq : n - t.nq - t.nk;
                    uint16_t* cache = static_cast<uint16_t*>(is_k ? t.cache_k : t.cache_v);
                    uint2 p;
                    p.x = Mma<T16>::pack2(y.x, y.y);
                    p.y = Mma<T16>::pack2(y.z, y.w);
                    *reinterpret_cast<uint2*>(cache + ((size_t)b * t.max_seq + pos) * (size_t)t.nk + cc) = p;
                }
            }
        }
    }
}

// Tile shapes: wave grid, accumulator tiles per wave, LDS ring slots (NS - 1 stages of
// loads in flight).
template <int BM, int BN> struct BigShape;
template <> struct BigShape<256, 256> { static constexpr int WGN = 2; };   // gemm_pp_kernel: 4 x 2 waves of 64 x 128
template <> struct BigShape<128, 128> { static constexpr int WGN = 4, TN = 2, NS = 3; };   // 2 x 4 waves of 64 x 32; 3 x 32 KB

template <typename T16, int BM, int BN, int EPI>
__global__ __launch_bounds__(512) void gemm_big_kernel(GemmArgs a, int n_tm, int n_tn) {
    static_assert(BM == 128, "the 256-row tile runs gemm_pp_kernel");
    typedef typename Mma<T16>::v8 v8_t;
    constexpr int BK = 64;                                 // K elements per stage (128 B a row)
    constexpr int WGN = BigShape<BM, BN>::WGN, TM = 4, TN = BigShape<BM, BN>::TN, WM = 64, WN = BN / WGN;
    constexpr int A_INS = BM / 64, B_INS = BN / 64;      // 8-row load instructions per wave
    constexpr int NS = BigShape<BM, BN>::NS;
    constexpr int kWait = (NS - 2) * (A_INS + B_INS);    // loads of the later stages in flight
    constexpr int kSlot = (BM + BN) * BK;                  // elements of one ring slot (A then B)
    constexpr uint32_t kSlotBytes = kSlot * 2;
    __shared__ __attribute__((aligned(1024))) uint16_t ring[NS * kSlot];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WGN, wn = wid % WGN;
    int tile_m, tile_n;
    if (!tile_of(blockIdx.x, n_tm, n_tn, tile_m, tile_n)) return;
    const int m0 = tile_m * BM;

    // Loads: one instruction fills 8 rows x 128 B; lane -> row lane / 8 of them and LDS chunk
    // lane % 8, which holds the row's global chunk (lane % 8) ^ (row % 8) (rows start at
    // multiples of 8).  Instruction i of wave w covers rows (INS * w + i) * 8 ...
    const int lrow = lane >> 3, lchunk = (lane & 7) ^ (lane >> 3);
    const uint16_t* ap[A_INS];
    const uint16_t* bp[B_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        const int gm = min(m0 + (A_INS * wid + i) * 8 + lrow, a.M - 1);
        ap[i] = static_cast<const uint16_t*>(a.a) + (size_t)gm * a.lda + lchunk * 8;
    }
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
        bool ok = true;
        bp[i] = b_row_ptr<BN, WGN, EPI>(a, tile_n, (B_INS * wid + i) * 8 + lrow, ok) + lchunk * 8;
    }
    const int nk_all = a.K / BK;
    const int kt0 = (int)((int64_t)nk_all * blockIdx.z / gridDim.z);
    const int kt1 = (int)((int64_t)nk_all * (blockIdx.z + 1) / gridDim.z);

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // This lane's fragment 0 of a slot for the K half h of a stage: row * 128 +
    // ((4h + g) ^ (row % 8)) * 16 bytes, row = (first row of the wave) + lane % 16; fragment i
    // sits 16 rows (2 KB) further with the same chunk.
    const int fr = lane & 15, g = lane >> 4;
    const uint32_t lr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)ring));
    const uint32_t fa[2] = {lr + (wm * WM + fr) * 128 + ((g ^ (fr & 7)) << 4),
                            lr + (wm * WM + fr) * 128 + (((4 + g) ^ (fr & 7)) << 4)};
    const uint32_t fb[2] = {lr + (BM + wn * WN + fr) * 128 + ((g ^ (fr & 7)) << 4),
                            lr + (BM + wn * WN + fr) * 128 + (((4 + g) ^ (fr & 7)) << 4)};

    auto issue = [&](int kt, uint16_t* slot) {
#pragma unroll
        for (int i = 0; i < A_INS; ++i)
            __builtin_amdgcn_global_load_lds((gbl_void_t*)(ap[i] + (size_t)kt * BK),
                                             (lds_void_t*)(slot + (A_INS * wid + i) * 8 * BK), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < B_INS; ++i)
            __builtin_amdgcn_global_load_lds((gbl_void_t*)(bp[i] + (size_t)kt * BK),
                                             (lds_void_t*)(slot + BM * BK + (B_INS * wid + i) * 8 * BK), 16, 0, 0);
    };
    auto compute = [&](uint32_t va, uint32_t vb) {
        // Fragment reads go out in asm blocks that wait for their own results: the compiler
        // then sees no LDS read it would have to order after the ring's DMA writes (it cannot
        // tell the slots apart across the loop and would drain every load).  The four A and
        // two B fragments of the K half, then its 8 MFMAs.
        static_assert(TM == 4 && TN == 2, "4 x 2 fragments");
        u32x4_t ra[TM], rb[TN];
        asm volatile(
            "ds_read_b128 %0, %6\n\t"
            "ds_read_b128 %1, %6 offset:2048\n\t"
            "ds_read_b128 %2, %6 offset:4096\n\t"
            "ds_read_b128 %3, %6 offset:6144\n\t"
            "ds_read_b128 %4, %7\n\t"
            "ds_read_b128 %5, %7 offset:2048\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(ra[0]), "=&v"(ra[1]), "=&v"(ra[2]), "=&v"(ra[3]), "=&v"(rb[0]), "=&v"(rb[1])
            : "v"(va), "v"(vb)
            : "memory");
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) {
            const v8_t bf = __builtin_bit_cast(v8_t, rb[jj]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[i][jj] = Mma<T16>::mma(__builtin_bit_cast(v8_t, ra[i]), bf, acc[i][jj]);
        }
    };

    // Prologue: stages 0..NS-2 (past the end: duplicates of the last stage, so every step has
    // the same number of loads outstanding).
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) issue(min(kt0 + i, kt1 - 1), ring + i * kSlot);

    // Step for stage kt held in slot S: wait for this wave's loads of that stage (those of
    // the NS - 2 later stages may stay in flight) and for its LDS reads of the previous
    // slot, barrier (now every wave's are done), refill the previous slot with stage
    // kt + NS - 1, compute both K halves of the stage.
    for (int kt = kt0; kt < kt1; kt += NS) {
#pragma unroll
        for (int S = 0; S < NS; ++S) {
            if (kt + S < kt1) {
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kWait) : "memory");
                issue(min(kt + S + NS - 1, kt1 - 1), ring + ((S + NS - 1) % NS) * kSlot);
                compute(fa[0] + S * kSlotBytes, fb[0] + S * kSlotBytes);
                compute(fa[1] + S * kSlotBytes, fb[1] + S * kSlotBytes);
            }
        }
    }
    // drain the duplicate tail loads; the nops keep the epilogue's reads of the accumulators
    // clear of the last asm MFMAs (the compiler cannot see their latency)
    asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    if (gridDim.z > 1) {
        // split K: raw fp32 tile of this split, [z][M][B row] with B rows n_tn * BN wide
        const int rq = (lane >> 4) * 4;
        const size_t ldp = (size_t)n_tn * BN;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int p = tile_n * BN + wn * WN + j * 16 + fr;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = m0 + wm * WM + i * 16 + rq + e;
                    if (m < a.M) a.part[((size_t)blockIdx.z * a.M + m) * ldp + p] = acc[i][j][e];
                }
            }
        return;
    }
    epilogue<T16, BN, WGN, TM, TN, EPI>(a, acc, m0, tile_n, wm, wn, lane);
}

// 256 x 256 tile with K in stages of 64 (the 256-row tile of both the long and the short
// path).  Same wave grid and accumulators as gemm_big_kernel<256> (8 waves as 4 x 2 of
// 64 x 128), but a stage row is 128 bytes, a whole cache line: one load instruction fills 8
// rows x 128 B, where 32-element stages fill 16 rows x 64 B and need twice the L2 requests for
// the same bytes (the request rate, not the bytes, bounded the 32-element ring).
//
// LDS: an A ring of 3 slots and a B ring of 2, 32 KB each (160 KB).  Waves w and w + 4 share a
// SIMD; group 0 (waves 0..3) computes A rows 0..127 of the tile and group 1 rows 128..255, so
// each group reads, and itself loads, only its half of an A slot, while both read every B row.
// Every wave takes each half-stage u (stage u / 2, K elements 32 (u % 2) .. + 31 of it) as a
// memory phase (its 12 fragments into registers, then 4 ring loads: B of stage u / 2 + 1 on
// even u, its group's A half of stage u / 2 + 2 on odd u) and then a compute phase (32 MFMAs),
// with a barrier after each phase; group 1 runs one phase behind group 0, so on each SIMD one
// wave issues MFMAs while the other reads LDS.  A slot is refilled only after every reader
// has finished with its previous stage (B: both groups' last reads are one and two phases
// before the refills; A: the group's own last read is two phases before), and each wave waits
// at the end of half-stage 2Y + 1 for all its loads but the newest batch, so stage Y + 1 is
// complete in every wave before the barrier that opens its first read.
template <typename T16, int EPI>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmArgs a, int n_tm, int n_tn) {
    typedef typename Mma<T16>::v8 v8_t;
    constexpr int BM = 256, BN = kBigBN, BK = 64, WGN = 2, TM = 4, TN = 8, WM = 64, WN = BN / WGN;
    constexpr int kSlot = 256 * BK;          // elements of one A or B slot (256 rows x 128 B)
    constexpr int NA = 3, NB = 2;
    __shared__ __attribute__((aligned(1024))) uint16_t ring[(NA + NB) * kSlot];
    uint16_t* const aring = ring;
    uint16_t* const bring = ring + NA * kSlot;

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WGN, wn = wid % WGN;
    const int grp = __builtin_amdgcn_readfirstlane(wid) >> 2;
    int tile_m, tile_n;
    if (!tile_of(blockIdx.x, n_tm, n_tn, tile_m, tile_n)) return;
    const int m0 = tile_m * BM;

    // Loads: lane -> row lane / 8 of the instruction's 8 rows and LDS chunk lane % 8, which
    // holds the row's global chunk (lane % 8) ^ (row % 8) (rows start at multiples of 8).
    const int lrow = lane >> 3, lchunk = (lane & 7) ^ (lane >> 3);
    const uint16_t* ap[4];
    const uint16_t* bp[4];
    int a_dst[4], b_dst[4];      // first row of each load instruction, as slot element offsets
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r0 = grp * 128 + ((wid & 3) * 4 + i) * 8;
        const int gm = min(m0 + r0 + lrow, a.M - 1);
        ap[i] = static_cast<const uint16_t*>(a.a) + (size_t)gm * a.lda + lchunk * 8;
        a_dst[i] = r0 * BK;
        const int rb = (wid * 4 + i) * 8;
        bool ok = true;
        bp[i] = b_row_ptr<BN, WGN, EPI>(a, tile_n, rb + lrow, ok) + lchunk * 8;
        b_dst[i] = rb * BK;
    }
    const int nk_all = a.K / BK;
    const int kt0 = (int)((int64_t)nk_all * blockIdx.z / gridDim.z);
    const int kt1 = (int)((int64_t)nk_all * (blockIdx.z + 1) / gridDim.z);
    const int n = kt1 - kt0;
    auto issue_a = [&](int kt, int slot) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((gbl_void_t*)(ap[i] + (size_t)kt * BK),
                                             (lds_void_t*)(aring + slot * kSlot + a_dst[i]), 16, 0, 0);
    };
    auto issue_b = [&](int kt, int slot) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds((gbl_void_t*)(bp[i] + (size_t)kt * BK),
                                             (lds_void_t*)(bring + slot * kSlot + b_dst[i]), 16, 0, 0);
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // This lane's fragment 0 in a slot, half-stage h: row * 128 + ((4h + g) ^ (row % 8)) * 16
    // bytes, row = (first row of the wave) + lane % 16; fragment i sits 16 rows (2 KB) further
    // with the same chunk (the rows differ by multiples of 8).
    const int fr = lane & 15, g = lane >> 4;
    const uint32_t la = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)aring));
    const uint32_t lb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)bring));
    const uint32_t fa0 = la + (wm * WM + fr) * 128 + ((g ^ (fr & 7)) << 4);
    const uint32_t fa1 = la + (wm * WM + fr) * 128 + (((4 + g) ^ (fr & 7)) << 4);
    const uint32_t fb0 = lb + (wn * WN + fr) * 128 + ((g ^ (fr & 7)) << 4);
    const uint32_t fb1 = lb + (wn * WN + fr) * 128 + (((4 + g) ^ (fr & 7)) << 4);

    auto half_stage = [&](uint32_t va, uint32_t vb, bool odd, int next_kt, int next_slot) {
        u32x4_t fa[TM], fb[TN];
        asm volatile(
            "ds_read_b128 %0, %12\n\t"
            "ds_read_b128 %1, %12 offset:2048\n\t"
            "ds_read_b128 %2, %12 offset:4096\n\t"
            "ds_read_b128 %3, %12 offset:6144\n\t"
            "ds_read_b128 %4, %13\n\t"
            "ds_read_b128 %5, %13 offset:2048\n\t"
            "ds_read_b128 %6, %13 offset:4096\n\t"
            "ds_read_b128 %7, %13 offset:6144\n\t"
            "ds_read_b128 %8, %13 offset:8192\n\t"
            "ds_read_b128 %9, %13 offset:10240\n\t"
            "ds_read_b128 %10, %13 offset:12288\n\t"
            "ds_read_b128 %11, %13 offset:14336\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(fa[0]), "=&v"(fa[1]), "=&v"(fa[2]), "=&v"(fa[3]), "=&v"(fb[0]), "=&v"(fb[1]),
              "=&v"(fb[2]), "=&v"(fb[3]), "=&v"(fb[4]), "=&v"(fb[5]), "=&v"(fb[6]), "=&v"(fb[7])
            : "v"(va), "v"(vb)
            : "memory");
        if (odd) {
            issue_a(next_kt, next_slot);
            // all of this wave's loads but the newest batch (A of stage Y + 2) are in
            if (grp) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        } else {
            issue_b(next_kt, next_slot);
        }
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const v8_t bf = __builtin_bit_cast(v8_t, fb[j]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[i][j] = Mma<T16>::mma(__builtin_bit_cast(v8_t, fa[i]), bf, acc[i][j]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (odd && !grp) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // Prologue: A(0), B(0), A(1) (past the end: duplicates of the last stage, so every wave
    // always has the same loads outstanding); wait for A(0) and B(0).
    issue_a(kt0, 0);
    issue_b(kt0, 0);
    issue_a(min(kt0 + 1, kt1 - 1), 1);
    asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    if (grp) asm volatile("s_barrier" ::: "memory");
    int sa = 0, sb = 0;     // slots of stage Y
    for (int Y = 0; Y < n; ++Y) {
        const int sa2 = sa == 0 ? 2 : sa - 1;   // slot of stage Y + 2: (Y + 2) % 3
        half_stage(fa0 + sa * (kSlot * 2), fb0 + sb * (kSlot * 2), false, min(kt0 + Y + 1, kt1 - 1), sb ^ 1);
        half_stage(fa1 + sa * (kSlot * 2), fb1 + sb * (kSlot * 2), true, min(kt0 + Y + 2, kt1 - 1), sa2);
        sa = sa == 2 ? 0 : sa + 1;
        sb ^= 1;
    }
    if (!grp) asm volatile("s_barrier" ::: "memory");
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");    // the duplicate tail loads
    if (gridDim.z > 1) {
        // split K: raw fp32 tile of this split, [z][M][B row] with B rows n_tn * BN wide
        const int rq = (lane >> 4) * 4;
        const size_t ldp = (size_t)n_tn * BN;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int p = tile_n * BN + wn * WN + j * 16 + fr;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int m = m0 + wm * WM + i * 16 + rq + e;
                    if (m < a.M) a.part[((size_t)blockIdx.z * a.M + m) * ldp + p] = acc[i][j][e];
                }
            }
        return;
    }
    if constexpr (EPI != EPI_STORE) {
        static_assert((NA + NB) * kSlot >= 8 * 64 * 64 * 2, "16 KB of ring per wave");
        epilogue_staged<T16, EPI>(a, acc, m0, tile_n, wm, wn, lane, reinterpret_cast<float*>(ring) + wid * 64 * 64);
    } else {
        epilogue<T16, BN, WGN, TM, TN, EPI>(a, acc, m0, tile_n, wm, wn, lane);
    }
}

// K splits for a short prefill (M <= kShortRows) on the LDS-ring kernels: about one
// workgroup per CU, at least kMinSplitK K elements (4 stages) per split, partials within the
// workspace.
constexpr int kShortRows = 512;
constexpr int kMinSplitK = 256;

// Tile width of the 128-row short-prefill kernel: 128 columns.  Against 256-column tiles
// (measured on the 128-row 7B prefill, 5.35 -> 4.97 ms) the [w1; w3] product needs no K split
// (172 tiles, its SiLU gate applied in the kernel's own epilogue, no reduce pass), q/k/v two
// splits instead of five and wo / w2 eight instead of sixteen, so half or less of the fp32
// partials are written and read back.
constexpr int kShortBN = 128;

template <typename T16, int BM, int BN, int EPI>
hipError_t launch_big(const GemmArgs& a, hipStream_t s) {
    const int ncols = (EPI == EPI_SWIGLU) ? BN / 2 : BN;
    const int n_tn = (a.N + ncols - 1) / ncols, n_tm = (a.M + BM - 1) / BM;
    const int per_xcd = (n_tn * n_tm + kXcds - 1) / kXcds;
    const size_t ldp = (size_t)n_tn * BN;
    int splits = 1;
    if (a.M <= kShortRows && a.part && (EPI == EPI_QKV || EPI == EPI_RESID || EPI == EPI_SWIGLU)) {
        // one workgroup per CU (its LDS ring takes most of the CU), all in one round
        const int tiles = n_tn * n_tm;
        splits = std::max(1, 256 / tiles);
        splits = std::min(splits, std::max(1, a.K / kMinSplitK));
        splits = std::min(splits, kMaxBigSplit);
        while (splits > 1 && (size_t)splits * a.M * ldp > a.part_cap) --splits;
    }
    if (a.deferred) *a.deferred = 0;
    if constexpr (BM == 256) {
        static_assert(BN == kBigBN, "the 256-row tile is 256 x 256");
        launch_kernel((gemm_pp_kernel<T16, EPI>), dim3(per_xcd * kXcds, 1, splits), dim3(512), 0, s, a, n_tm, n_tn);
    } else {
        launch_kernel((gemm_big_kernel<T16, BM, BN, EPI>), dim3(per_xcd * kXcds, 1, splits), dim3(512), 0, s, a,
                      n_tm, n_tn);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const size_t n = (size_t)a.M * a.N;
    const dim3 rgrid((unsigned)((n + 255) / 256));
    if constexpr (EPI == EPI_RESID) {
        if (a.deferred && ldp == (size_t)a.N && splits <= kMaxNormFold) {   // [splits][M][N]: the next norm folds them
            *a.deferred = splits;
            return hipSuccess;
        }
        launch_kernel(splitk_reduce_kernel, rgrid, dim3(256), 0, s, a.part, splits, a.M, a.N,
                      (int64_t)ldp, a.resid, a.ldr);
    } else if constexpr (EPI == EPI_SWIGLU) {
        launch_kernel(swiglu_reduce_kernel<T16>, rgrid, dim3(256), 0, s, a.part, splits, a.M, a.N,
                      (int64_t)ldp, BN, BN / BigShape<BM, BN>::WGN, static_cast<uint16_t*>(a.out16),
                      a.ldo16);
    } else {
        return launch_rope_scatter_parts(a.part, splits, (int64_t)ldp, a.M, a.qkv, s, a.wtype);
    }
    return hipGetLastError();
}

template <typename T16, int EPI>
hipError_t launch_epi(const GemmArgs& a, hipStream_t s) {
    // Small M: narrow register-staged tiles.
    if (a.M <= 64) return launch_tile<T16, 64, 64, 2, 2, EPI>(a, s);
    // Short prefills: the weights are the traffic; the LDS-ring kernel with K split so about
    // one workgroup per CU streams them, the epilogue applied by a reduce pass.
    if constexpr (EPI == EPI_QKV || EPI == EPI_RESID || EPI == EPI_SWIGLU) {
        if (a.M <= kShortRows && a.part) {
            if (a.M <= 128) return launch_big<T16, 128, kShortBN, EPI>(a, s);
            return launch_big<T16, 256, kBigBN, EPI>(a, s);
        }
    }
    if (a.M <= 256) return launch_tile<T16, 128, 64, 2, 2, EPI>(a, s);
    if (a.M <= 2048) return launch_tile<T16, 128, 128, 2, 2, EPI>(a, s);
    if constexpr (EPI == EPI_QKV || EPI == EPI_RESID || EPI == EPI_SWIGLU) {
        // 256 x 256 tiles run one per CU, in rounds of kCUs.  When the last round would be
        // nearly empty, the last one or two tile rows (at most kShortRows rows) go to the
        // split-K short path instead, which spreads them over every CU; the choice follows a
        // cost estimate in rounds (the split rows' share of a round, plus a fixed charge for
        // the extra launches and the reduce pass).
        if (a.part) {
            const int ncols = (EPI == EPI_SWIGLU) ? kBigBN / 2 : kBigBN;
            const int n_tn = (a.N + ncols - 1) / ncols, n_tm = (a.M + 255) / 256;
            auto rounds = [&](int tiles) { return (double)((tiles + kCUs - 1) / kCUs); };
            double best = rounds(n_tm * n_tn);
            int best_t = 0;
            for (int t = 1; t <= 2; ++t) {
                const int M1 = (n_tm - t) * 256, M2 = a.M - M1;
                if (M1 <= 2048 || M2 > kShortRows) continue;
                const double r = rounds((n_tm - t) * n_tn) + 1.3 * M2 / 256.0 * n_tn / kCUs + 0.15;
                if (r < best) {
                    best = r;
                    best_t = t;
                }
            }
            if (best_t > 0) {
                // two launches over row ranges: each adds its result to resid itself (deferred
                // partials must cover every row of the product in one [splits][M][N] block)
                if (a.deferred) *a.deferred = 0;
                const int M1 = (n_tm - best_t) * 256, M2 = a.M - M1;
                GemmArgs a1 = a;
                a1.M = M1;
                a1.deferred = nullptr;
                const hipError_t e = launch_big<T16, 256, kBigBN, EPI>(a1, s);
                if (e != hipSuccess) return e;
                GemmArgs a2 = a;
                a2.M = M2;
                a2.deferred = nullptr;
                a2.a = static_cast<const uint16_t*>(a.a) + (size_t)M1 * a.lda;
                if constexpr (EPI == EPI_RESID) a2.resid = a.resid + (size_t)M1 * a.ldr;
                if constexpr (EPI == EPI_SWIGLU) a2.out16 = static_cast<uint16_t*>(a.out16) + (size_t)M1 * a.ldo16;
                if constexpr (EPI == EPI_QKV) a2.qkv.row0 = a.qkv.row0 + M1;
                return M2 <= 128 ? launch_big<T16, 128, kShortBN, EPI>(a2, s)
                                 : launch_big<T16, 256, kBigBN, EPI>(a2, s);
            }
        }
    }
    return launch_big<T16, 256, kBigBN, EPI>(a, s);
}

template <typename T16>
hipError_t launch_typed(int epi, const GemmArgs& a, hipStream_t s) {
    switch (epi) {
        case EPI_QKV: return launch_epi<T16, EPI_QKV>(a, s);
        case EPI_RESID: return launch_epi<T16, EPI_RESID>(a, s);
        case EPI_SWIGLU: return launch_epi<T16, EPI_SWIGLU>(a, s);
        default: return launch_epi<T16, EPI_STORE>(a, s);
    }
}

}  // namespace

hipError_t launch_gemm(int epi, const GemmArgs& a, hipStream_t s) {
    switch (a.wtype) {
        case kStoreBf16: return launch_typed<bf16>(epi, a, s);
        case kStoreF16: return launch_typed<f16>(epi, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace llk
