// Round kernels around the head matmul: n-gram drafter, greedy accept, RMSNorm.
#include "sv_device.h"
#include "sv_internal.h"

#include "../../include/specverify.h"

namespace sv {

namespace {

constexpr int kProposeThreads = 1024;
constexpr int kChunk = 8192;                 // stream ids staged in LDS per pass
constexpr int kHalo = SV_MAX_NGRAM;          // ids before the chunk a match may reach back to

// n-gram prompt lookup ("Stream C - Speculative decoding", the delta: the last m ids of the
// stream index their most recent continuation; "Spec-decode on GDN hybrids", harness
// lessons: the stream ends in the pending anchor, so drafts continue past it).
// For every end position e <= len-2 a thread computes the match length l(e) of the
// stream's suffix ending at e (capped at nmax).  "First n from nmax down with a match,
// latest occurrence" is the lexicographic maximum of (l(e), e); one 64-bit max-reduction
// finds it.  The stream is staged through LDS in chunks so the scan reads HBM once.
__global__ __launch_bounds__(kProposeThreads) void propose_kernel(const int32_t* __restrict__ tokens,
                                                                  int cap, int32_t* __restrict__ state,
                                                                  int nmax, int K, int32_t* __restrict__ drafts) {
    __shared__ int32_t tk[kHalo + kChunk];
    __shared__ unsigned long long wbest[kProposeThreads / kWave];
    const int tid = threadIdx.x;
    int len = state[SV_STATE_LEN];
    if (len < 0 || len > cap) {              // corrupt state: never read past the buffer
        if (tid == 0) state[SV_STATE_FLAGS] |= SV_FLAG_CAPACITY;
        len = 0;
    }

    int32_t suf[SV_MAX_NGRAM];
#pragma unroll
    for (int i = 0; i < SV_MAX_NGRAM; ++i) suf[i] = (i < nmax && len - 1 - i >= 0) ? tokens[len - 1 - i] : -1;

    unsigned long long best = 0;
    for (int base = 0; base < len - 1; base += kChunk) {
        __syncthreads();
        for (int t = tid; t < kHalo + kChunk; t += kProposeThreads) {
            const int idx = base - kHalo + t;
            tk[t] = (idx >= 0 && idx < len) ? tokens[idx] : 0;
        }
        __syncthreads();
        const int end = min(base + kChunk, len - 1);     // e in [base, end)
        for (int e = base + tid; e < end; e += kProposeThreads) {
            int l = 0;
#pragma unroll
            for (int i = 0; i < SV_MAX_NGRAM; ++i) {
                if (l == i && i < nmax && e - i >= 0 && tk[e - i - base + kHalo] == suf[i]) l = i + 1;
            }
            if (l > 0) {
                const unsigned long long key = ((unsigned long long)l << 32) | (unsigned)e;
                best = key > best ? key : best;
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(best, off, 64);
        best = o > best ? o : best;
    }
    if ((tid & 63) == 0) wbest[tid >> 6] = best;
    __syncthreads();
    if (tid < kWave) {
        unsigned long long b = tid < kProposeThreads / kWave ? wbest[tid] : 0ull;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const unsigned long long o = __shfl_xor(b, off, 64);
            b = o > b ? o : b;
        }
        const int nused = (int)(b >> 32);
        const int e = (int)(b & 0xffffffffu);
        if (tid < K) {
            const int p = e + 1 + tid;
            drafts[tid] = (nused > 0 && p <= len - 1) ? tokens[p] : -1;
        }
        if (tid == 0) {
            const int nv = nused > 0 ? min(K, len - 1 - e) : 0;
            state[SV_STATE_NVALID] = nv;
            state[SV_STATE_NUSED] = nused;
        }
    }
}

// Greedy accept, one wave ("Stream C - Speculative decoding", the delta and control-logic
// proof; "Spec-decode on GDN hybrids", hybrid state discipline): lane i compares d_{i+1}
// with the greedy id of window row i, a ballot finds the first miss j, the accepted drafts
// and argmax[j] (correction or bonus) are appended and len advances by 1 + j.
__global__ __launch_bounds__(kWave) void accept_kernel(const int32_t* __restrict__ argmax,
                                                       const int32_t* __restrict__ drafts, int K,
                                                       int32_t* __restrict__ tokens, int cap,
                                                       int32_t* __restrict__ state) {
    const int lane = threadIdx.x;
    const int len = state[SV_STATE_LEN];
    if (len + K + 1 > cap || len < 0) {
        if (lane == 0) state[SV_STATE_FLAGS] |= SV_FLAG_CAPACITY;
        return;
    }
    int d = -1, a = -2;
    if (lane < K) { d = drafts[lane]; a = argmax[lane]; }
    const unsigned long long hit = __ballot(lane < K && d >= 0 && d == a);
    const int j = __builtin_ctzll(~hit);                 // <= K: bit K is never set
    if (lane < j) tokens[len + lane] = d;
    if (lane == j) tokens[len + j] = argmax[j];
    if (lane == 0) {
        state[SV_STATE_LEN] = len + 1 + j;
        state[SV_STATE_J] = j;
        state[SV_STATE_ROUNDS] += 1;
        state[SV_STATE_SUMJ] += j;
        state[SV_STATE_HIST + j] += 1;
    }
}

// y = fp16(x / sqrt(mean(x^2) + eps)) per row, fp32 math, fixed reduction order.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x, int H, float eps,
                                                      uint16_t* __restrict__ y) {
    const int s = blockIdx.x;
    const uint16_t* xr = x + (size_t)s * H;
    float acc = 0.f;
    for (int k = threadIdx.x; k < H; k += 256) {
        const float v = h2f(xr[k]);
        acc = __builtin_fmaf(v, v, acc);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    const float tot = (part[0] + part[1]) + (part[2] + part[3]);
    const float r = 1.0f / sqrtf(tot / (float)H + eps);
    for (int k = threadIdx.x; k < H; k += 256) y[(size_t)s * H + k] = f2h(h2f(xr[k]) * r);
}

}  // namespace

hipError_t launch_propose(const int32_t* tokens, int cap, int32_t* state, int nmax, int K, int32_t* drafts,
                          hipStream_t stream) {
    hipLaunchKernelGGL(propose_kernel, dim3(1), dim3(kProposeThreads), 0, stream, tokens, cap, state, nmax, K,
                       drafts);
    return hipGetLastError();
}

hipError_t launch_accept(const int32_t* argmax, const int32_t* drafts, int K, int32_t* tokens, int cap,
                         int32_t* state, hipStream_t stream) {
    hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(kWave), 0, stream, argmax, drafts, K, tokens, cap, state);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const uint16_t* x, int S, int H, float eps, uint16_t* y, hipStream_t stream) {
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(S), dim3(256), 0, stream, x, H, eps, y);
    return hipGetLastError();
}

}  // namespace sv
