// Temperature + top-p ("nucleus") draw of one token per row, on the device.
//
// The method ([AG] 8.5, temperature > 0; [ST] "Sampling, Stopping, and the Chat Template"):
// probabilities p = softmax(logits / temperature); sort descending; drop the tokens beyond
// the cumulative top-p mass; renormalise; draw one token.  Readings: a token is dropped
// when the mass sorted before it exceeds top_p; equal probabilities sort by lower index; the
// draw is the inverse CDF in sorted order at a uniform u in [0, 1) that the caller passes in.
//
// No sort is materialised.  Every token gets a 64-bit key, (~bits(p) << 32) | index, whose
// ascending order is the sorted order (p >= 0, so its bit pattern orders like its value).
// With f(K) = the mass of the tokens whose key is below K, a token is kept iff
// f(key) <= top_p, so the last kept token is the largest K with f(K) <= top_p (one binary
// search over the key space), and the drawn token is the largest K with
// f(K) <= u * (kept mass) (a second).  Each step of a search is one workgroup sum; a row's
// probabilities stay in registers (one 512-thread workgroup per row, 64 per thread).
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;
constexpr int kPerThread = kMaxSampleVocab / kThreads;

// Workgroup sum / max, identical in every thread (the waves' partials are combined in the
// same order everywhere).
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    float t = 0.f;
#pragma clang loop unroll(full)
    for (int w = 0; w < kWaves; ++w) t += red[w];
    __syncthreads();
    return t;
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma clang loop unroll(full)
    for (int o = kWave / 2; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    float t = red[0];
#pragma clang loop unroll(full)
    for (int w = 1; w < kWaves; ++w) t = fmaxf(t, red[w]);
    __syncthreads();
    return t;
}

__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* red) {
#pragma clang loop unroll(full)
    for (int o = kWave / 2; o >= 1; o >>= 1) {
        const uint64_t w = __shfl_xor(v, o, kWave);
        v = w > v ? w : v;
    }
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    uint64_t t = red[0];
#pragma clang loop unroll(full)
    for (int w = 1; w < kWaves; ++w) t = red[w] > t ? red[w] : t;
    __syncthreads();
    return t;
}

__global__ __launch_bounds__(kThreads) void sample_top_p_kernel(const float* logits, int vocab, int64_t stride,
                                                                float inv_temp, float top_p, const float* uniform,
                                                                int32_t* out, float* logprob) {
    __shared__ float red[kWaves];
    __shared__ uint64_t redk[kWaves];
    const int tid = threadIdx.x;
    const float* x = logits + (size_t)blockIdx.x * stride;

    float p[kPerThread];
    float mx = -INFINITY;
#pragma clang loop unroll(full)
    for (int j = 0; j < kPerThread; ++j) {
        const int i = tid + kThreads * j;
        p[j] = i < vocab ? x[i] : -INFINITY;
        mx = fmaxf(mx, p[j]);
    }
    mx = block_max(mx, red);
    // softmax of logits / temperature (its max is mx / temperature: temperature > 0), and the
    // plain softmax's normaliser for the log-prob
    const float mz = mx * inv_temp;
    float s = 0.f, sr = 0.f;
#pragma clang loop unroll(full)
    for (int j = 0; j < kPerThread; ++j) {
        const int i = tid + kThreads * j;
        float e = 0.f;
        if (i < vocab) {
            e = __expf(p[j] * inv_temp - mz);
            sr += __expf(p[j] - mx);
        }
        p[j] = e;
        s += e;
    }
    s = block_sum(s, red);
    sr = block_sum(sr, red);
    // Each element is held as the high half of its sort key, ~bits(p): p is recovered as
    // the float with bits ~hi, and (hi, index) compared as two 32-bit halves gives the sort
    // order (64-bit keys for all 64 elements would not fit the register budget).  Entries past
    // the vocabulary hold p = 0 and an index >= vocab, so they rank after every token.
    const float inv_s = 1.f / s;
    uint32_t hi[kPerThread];
#pragma clang loop unroll(full)
    for (int j = 0; j < kPerThread; ++j) hi[j] = ~__float_as_uint(p[j] * inv_s);
    auto prob = [&](int j) __attribute__((always_inline)) { return __uint_as_float(~hi[j]); };
    auto below = [&](int j, uint64_t K) __attribute__((always_inline)) {
        const uint32_t i = (uint32_t)(tid + kThreads * j), khi = (uint32_t)(K >> 32), klo = (uint32_t)K;
        return hi[j] < khi || (hi[j] == khi && i < klo);
    };
    auto mass_below = [&](uint64_t K) __attribute__((always_inline)) {
        // the empty asm marks the keys as rewritten, so the compiler recomputes each p from
        // its key here instead of keeping a second register copy of all 64 across the search
#pragma clang loop unroll(full)
        for (int j = 0; j < kPerThread; ++j) asm volatile("" : "+v"(hi[j]));
        float a = 0.f;
#pragma clang loop unroll(full)
        for (int j = 0; j < kPerThread; ++j) a += below(j, K) ? prob(j) : 0.f;
        return block_sum(a, red);
    };
    // largest K in [lo, hi] with f(K) <= t, given f(lo) <= t (f is non-decreasing)
    auto search = [&](uint64_t lo, uint64_t top, float t) __attribute__((always_inline)) {
        while (lo < top) {
            const uint64_t mid = lo + (top - lo) / 2 + 1;
            if (mass_below(mid) <= t)
                lo = mid;
            else
                top = mid - 1;
        }
        return lo;
    };
    // the last kept token and the kept mass
    uint64_t kept_last;
    float kept_mass;
    if (top_p >= 1.f) {
        kept_last = ~0ull;
        float a = 0.f;
#pragma clang loop unroll(full)
        for (int j = 0; j < kPerThread; ++j) a += prob(j);
        kept_mass = block_sum(a, red);
    } else {
        kept_last = search(0, ~0ull, top_p);
        kept_mass = mass_below(kept_last + 1);
    }
    // inverse CDF at u * kept mass, within the kept tokens
    float u = uniform[blockIdx.x];
    u = fminf(fmaxf(u, 0.f), 0x1.fffffep-1f);
    const uint64_t k2 = search(0, kept_last, u * kept_mass);
    uint64_t best = 0;
#pragma clang loop unroll(full)
    for (int j = 0; j < kPerThread; ++j) {
        const int i = tid + kThreads * j;
        const uint64_t k = ((uint64_t)hi[j] << 32) | (uint32_t)i;
        if (i < vocab && k <= k2 && k > best) best = k;
    }
    best = block_max_u64(best, redk);
    if (tid == 0) {
        const int tok = (int)(uint32_t)(best & 0xffffffffu);
        out[blockIdx.x] = tok;
        if (logprob) logprob[blockIdx.x] = x[tok] - mx - __logf(sr);
    }
}

}  // namespace

hipError_t launch_sample_top_p(const float* logits, int bsz, int vocab, int64_t stride, float temperature,
                               float top_p, const float* uniform, int32_t* out, float* logprob, hipStream_t s) {
    launch_kernel(sample_top_p_kernel, dim3(bsz), dim3(kThreads), 0, s, logits, vocab, stride, 1.f / temperature,
                  top_p, uniform, out, logprob);
    return hipGetLastError();
}

}  // namespace llk
