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
                        t.q[(size_t)mm * t.nq + n] = round_bf16(v);
                    } else {
                        const bool is_k = n < t.nq + t.nk;
                        const int c = is_k ? n - t.nq : n - t.nq - t.nk;
                        uint16_t* cache = static_cast<uint16_t*>(is_k ? t.cache_k : t.cache_v);
                        cache[cache_row + c] = f32_to_bf16(v);
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
    out[(size_t)m * ldo + u] = f32_to_bf16(silu(g) * v);
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
                  a.part, splits, a.M, a.N, (int64_t)a.N, a.resid, a.ldr);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------------------
// LDS-ring variant: BM x 256 tiles (BM = 256: 8 waves as 4 x 2 of 64 x 128; BM = 128: 8 waves
// as 2 x 4 of 64 x 64), K in stages of 32 through an LDS ring (4 slots at BM = 256, 6 at 128)
// filled by global_load_lds_dwordx4 (global -> LDS without registers), loads issued NS - 1
// stages ahead.  Long prefills use it with the LDS-staged epilogue below; short ones (a few
// hundred rows, where the weights are the traffic) split K over gridDim.z so enough
// workgroups stream the weights: each split stores its raw fp32 tile [z][M][B row] and a
// reduce pass applies the epilogue.  A wave's load instruction fills 1 KB of LDS
// contiguously (lane i -> bytes 16i..16i+15), i.e. 16 rows x 4 chunks of a 64-byte row; each
// lane fetches the global chunk (chunk ^ swz(row)), so a fragment read of (row, chunk) finds
// it at slot chunk ^ swz(row) and the rows of a fragment land on distinct banks without
// padding.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr int kBigBN = 256, kBigBK = 32;

// The LDS serves a 16-byte read 8 lanes at a time from a 128-byte bank window; rows are 64
// bytes, so rows r and r + 2 share a window offset.  XOR-ing the chunk with (row / 2) % 4
// puts the 8 rows of a lane group on 8 distinct 16-byte slots (measured: the previous
// (row / 4) % 4 gave every fragment read a 2-way conflict).
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 3; }

// Tile shapes: wave grid, accumulator tiles per wave, LDS ring slots (NS - 1 stages of
// loads in flight).  The 128-row tile is for short prefills, where the weights are the
// traffic: its smaller A tile leaves room for a deeper ring.
// Eight MFMAs of one fragment group, c[i][jj] += a[i] * b[jj] (i < 4, jj < 2), with the two
// B fragment reads of the next group issued ahead of them and waited for at the end of the
// block: the reads are in flight while the MFMAs run, and no asm output is left pending.
// The accumulators chain MFMA to MFMA on the same registers (no wait states needed); the
// new fragments go to registers no MFMA of this block reads (early clobber).
__device__ __forceinline__ void mfma8_read2(f32x4& c00, f32x4& c10, f32x4& c20, f32x4& c30,
                                            f32x4& c01, f32x4& c11, f32x4& c21, f32x4& c31,
                                            const u32x4_t& a0, const u32x4_t& a1, const u32x4_t& a2,
                                            const u32x4_t& a3, const u32x4_t& b0, const u32x4_t& b1,
                                            u32x4_t& n0, u32x4_t& n1, uint32_t addr0, uint32_t addr1) {
    asm volatile(
        "ds_read_b128 %8, %10\n\t"
        "ds_read_b128 %9, %11\n\t"
        "v_mfma_f32_16x16x32_bf16 %0, %12, %16, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %13, %16, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %14, %16, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %15, %16, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %4, %12, %17, %4\n\t"
        "v_mfma_f32_16x16x32_bf16 %5, %13, %17, %5\n\t"
        "v_mfma_f32_16x16x32_bf16 %6, %14, %17, %6\n\t"
        "v_mfma_f32_16x16x32_bf16 %7, %15, %17, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "+v"(c00), "+v"(c10), "+v"(c20), "+v"(c30), "+v"(c01), "+v"(c11), "+v"(c21), "+v"(c31),
          "=&v"(n0), "=&v"(n1)
        : "v"(addr0), "v"(addr1), "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(b0), "v"(b1)
        : "memory");
}

// Epilogue of the 256 x 256 kernel through LDS.  A wave's accumulators (64 rows x 128
// columns, 4 consecutive rows of one column per lane and tile) go to its own 16 KB of the
// then idle ring as fp32, 64 columns per pass, and come back as 16-byte row chunks, 16 lanes
// to a row: the residual rows are read and written, and the q / K / V / gated rows written,
// in whole 256-byte segments rather than 4-byte pieces.  Chunks (4 floats) are XOR-swizzled
// by row so that both the column-wise writes and the row-wise reads spread over the banks.
// RoPE is applied on the row chunks: a lane holds two whole (even, odd) pairs.
template <int EPI>
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
                p.x = pack_bf16x2(v.x, v.y);
                p.y = pack_bf16x2(v.z, v.w);
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
                        float4{round_bf16(y.x), round_bf16(y.y), round_bf16(y.z), round_bf16(y.w)};
                } else {
                    const bool is_k = n < t.nq + t.nk;
                    const int cc = is_k ? n - t.nq : n - t.nq - t.nk;
                    uint16_t* cache = static_cast<uint16_t*>(is_k ? t.cache_k : t.cache_v);
                    uint2 p;
                    p.x = pack_bf16x2(y.x, y.y);
                    p.y = pack_bf16x2(y.z, y.w);
                    *reinterpret_cast<uint2*>(cache + ((size_t)b * t.max_seq + pos) * (size_t)t.nk + cc) = p;
                }
            }
        }
    }
}

template <int BM> struct BigShape;
template <> struct BigShape<256> { static constexpr int WGN = 2, TN = 8, NS = 4; };   // 4 x 2 waves of 64 x 128; 128 KB
template <> struct BigShape<128> { static constexpr int WGN = 4, TN = 4, NS = 6; };   // 2 x 4 waves of 64 x 64; 144 KB

template <int BM, int EPI>
__global__ __launch_bounds__(512) void gemm_big_kernel(GemmArgs a, int n_tm, int n_tn) {
    constexpr int BN = kBigBN, BKS = kBigBK;
    constexpr int WGN = BigShape<BM>::WGN, TM = 4, TN = BigShape<BM>::TN, WM = 64, WN = BN / WGN;
    constexpr int A_INS = BM / 128, B_INS = BN / 128;    // 16-row load instructions per wave
    constexpr int NS = BigShape<BM>::NS;
    constexpr int kWait = (NS - 2) * (A_INS + B_INS);    // loads of the later stages in flight
    constexpr int kSlot = (BM + BN) * BKS;                 // elements of one ring slot (A then B)
    // The fragment reads are asm blocks that wait for their own results, so the compiler
    // sees no LDS read it would have to order after the ring's DMA writes.
    __shared__ __attribute__((aligned(1024))) uint16_t ring[NS * kSlot];

    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WGN, wn = wid % WGN;
    int tile_m, tile_n;
    if (!tile_of(blockIdx.x, n_tm, n_tn, tile_m, tile_n)) return;
    const int m0 = tile_m * BM;

    // This lane's A rows and B rows (one per load instruction of the wave: rows
    // (INS * wid + i) * 16 + lane / 4 of the tile).
    const uint16_t* ap[A_INS];
    const uint16_t* bp[B_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        const int row = (A_INS * wid + i) * 16 + (lane >> 2);
        const int gc = (lane & 3) ^ swz(row);
        const int gm = min(m0 + row, a.M - 1);
        ap[i] = static_cast<const uint16_t*>(a.a) + (size_t)gm * a.lda + gc * 8;
    }
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
        const int row = (B_INS * wid + i) * 16 + (lane >> 2);
        const int gc = (lane & 3) ^ swz(row);
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
        for (int i = 0; i < A_INS; ++i)
            __builtin_amdgcn_global_load_lds((gbl_void_t*)(ap[i] + (size_t)kt * BKS),
                                             (lds_void_t*)(Ad + (A_INS * wid + i) * 16 * BKS), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < B_INS; ++i)
            __builtin_amdgcn_global_load_lds((gbl_void_t*)(bp[i] + (size_t)kt * BKS),
                                             (lds_void_t*)(Bd + (B_INS * wid + i) * 16 * BKS), 16, 0, 0);
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
        static_assert(TM == 4, "mfma8_read2 covers four A fragments");
        // groups 0 .. TN/2 - 2: MFMAs of group jg with group jg + 1's B reads in flight
#pragma unroll
        for (int jg = 0; jg + 1 < TN / 2; ++jg)
            mfma8_read2(acc[0][2 * jg], acc[1][2 * jg], acc[2][2 * jg], acc[3][2 * jg],
                        acc[0][2 * jg + 1], acc[1][2 * jg + 1], acc[2][2 * jg + 1], acc[3][2 * jg + 1],
                        ra[0], ra[1], ra[2], ra[3], rb[2 * jg], rb[2 * jg + 1], rb[2 * jg + 2], rb[2 * jg + 3],
                        bb + 2 * b_off[2 * jg + 2], bb + 2 * b_off[2 * jg + 3]);
        // last group
        constexpr int jl = TN / 2 - 1;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, rb[2 * jl + jj]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                acc[i][2 * jl + jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, ra[i]), bf, acc[i][2 * jl + jj], 0, 0, 0);
        }
    };

    // Prologue: stages 0..NS-2 (past the end: duplicates of the last stage, so every step has
    // the same number of loads outstanding).
#pragma unroll
    for (int i = 0; i < NS - 1; ++i) issue(min(kt0 + i, kt1 - 1), ring + i * kSlot, ring + i * kSlot + BM * BKS);

    // Step for stage kt held in slot S: wait for this wave's loads of that stage (those of the
    // NS - 2 later stages may stay in flight) and for its LDS reads of the previous slot,
    // barrier (now every wave's are done), refill the previous slot with stage kt + NS - 1,
    // compute.
    for (int kt = kt0; kt < kt1; kt += NS) {
#pragma unroll
        for (int S = 0; S < NS; ++S) {
            if (kt + S < kt1) {
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kWait) : "memory");
                uint16_t* prev = ring + ((S + NS - 1) % NS) * kSlot;
                issue(min(kt + S + NS - 1, kt1 - 1), prev, prev + BM * BKS);
                compute(ring + S * kSlot, ring + S * kSlot + BM * BKS);
            }
        }
    }
    // drain the duplicate tail loads; the nops keep the epilogue's reads of the accumulators
    // clear of the last asm MFMAs (the compiler cannot see their latency)
    asm volatile("s_waitcnt vmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    if (gridDim.z > 1) {
        // split K: raw fp32 tile of this split, [z][M][B row] with B rows n_tn * BN wide
        const int fr = lane & 15, rq = (lane >> 4) * 4;
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
    if constexpr (BM == 256 && EPI != EPI_STORE) {
        static_assert(TN == 8 && WN == 128 && NS * kSlot >= 8 * 64 * 64 * 2, "16 KB of ring per wave");
        epilogue_staged<EPI>(a, acc, m0, tile_n, wm, wn, lane, reinterpret_cast<float*>(ring) + wid * 64 * 64);
    } else {
        epilogue<BN, WGN, TM, TN, EPI>(a, acc, m0, tile_n, wm, wn, lane);
    }
}

// K splits for a short prefill (M <= kShortRows) on the LDS-ring kernel: about one
// workgroup per CU, at least 8 k-stages per split, partials within the workspace.
constexpr int kShortRows = 512;

template <int BM, int EPI>
hipError_t launch_big(const GemmArgs& a, hipStream_t s) {
    const int ncols = (EPI == EPI_SWIGLU) ? kBigBN / 2 : kBigBN;
    const int n_tn = (a.N + ncols - 1) / ncols, n_tm = (a.M + BM - 1) / BM;
    const int per_xcd = (n_tn * n_tm + kXcds - 1) / kXcds;
    const size_t ldp = (size_t)n_tn * kBigBN;
    int splits = 1;
    if (a.M <= kShortRows && a.part && (EPI == EPI_QKV || EPI == EPI_RESID || EPI == EPI_SWIGLU)) {
        // one workgroup per CU (its LDS ring takes most of the CU), all in one round
        const int tiles = n_tn * n_tm;
        splits = std::max(1, 256 / tiles);
        splits = std::min(splits, std::max(1, a.K / kBigBK / 8));
        splits = std::min(splits, kMaxBigSplit);
        while (splits > 1 && (size_t)splits * a.M * ldp > a.part_cap) --splits;
    }
    launch_kernel((gemm_big_kernel<BM, EPI>), dim3(per_xcd * kXcds, 1, splits), dim3(512), 0, s, a,
                  n_tm, n_tn);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const size_t n = (size_t)a.M * a.N;
    const dim3 rgrid((unsigned)((n + 255) / 256));
    if constexpr (EPI == EPI_RESID) {
        launch_kernel(splitk_reduce_kernel, rgrid, dim3(256), 0, s, a.part, splits, a.M, a.N,
                      (int64_t)ldp, a.resid, a.ldr);
    } else if constexpr (EPI == EPI_SWIGLU) {
        launch_kernel(swiglu_reduce_kernel, rgrid, dim3(256), 0, s, a.part, splits, a.M, a.N,
                      (int64_t)ldp, kBigBN, kBigBN / BigShape<BM>::WGN, static_cast<uint16_t*>(a.out16),
                      a.ldo16);
    } else {
        return launch_rope_scatter_parts(a.part, splits, (int64_t)ldp, a.M, a.qkv, s);
    }
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs& a, hipStream_t s) {
    // Small M: narrow register-staged tiles.
    if (a.M <= 64) return launch_tile<64, 64, 2, 2, EPI>(a, s);
    // Short prefills: the weights are the traffic; the LDS-ring kernel with K split so about
    // one workgroup per CU streams them, the epilogue applied by a reduce pass.
    if constexpr (EPI == EPI_QKV || EPI == EPI_RESID || EPI == EPI_SWIGLU) {
        if (a.M <= kShortRows && a.part) {
            if (a.M <= 128) return launch_big<128, EPI>(a, s);
            return launch_big<256, EPI>(a, s);
        }
    }
    if (a.M <= 256) return launch_tile<128, 64, 2, 2, EPI>(a, s);
    if (a.M <= 2048) return launch_tile<128, 128, 2, 2, EPI>(a, s);
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
                const int M1 = (n_tm - best_t) * 256, M2 = a.M - M1;
                GemmArgs a1 = a;
                a1.M = M1;
                const hipError_t e = launch_big<256, EPI>(a1, s);
                if (e != hipSuccess) return e;
                GemmArgs a2 = a;
                a2.M = M2;
                a2.a = static_cast<const uint16_t*>(a.a) + (size_t)M1 * a.lda;
                if constexpr (EPI == EPI_RESID) a2.resid = a.resid + (size_t)M1 * a.ldr;
                if constexpr (EPI == EPI_SWIGLU) a2.out16 = static_cast<uint16_t*>(a.out16) + (size_t)M1 * a.ldo16;
                if constexpr (EPI == EPI_QKV) a2.qkv.row0 = a.qkv.row0 + M1;
                return M2 <= 128 ? launch_big<128, EPI>(a2, s) : launch_big<256, EPI>(a2, s);
            }
        }
    }
    return launch_big<256, EPI>(a, s);
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
