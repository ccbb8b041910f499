// Standalone round kernels around the head matmul: n-gram drafter, greedy accept, RMSNorm.
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_tail.h"

#include "../../include/specverify.h"

namespace sv {

namespace {

constexpr int kProposeThreads = 1024;
constexpr int kChunk = 8192;                 // stream ids staged in LDS per pass

__global__ __launch_bounds__(kProposeThreads) void propose_kernel(const int32_t* __restrict__ tokens,
                                                                  int cap, int32_t* __restrict__ state,
                                                                  int nmax, int K, int32_t* __restrict__ drafts) {
    __shared__ int32_t tk[kHalo + kChunk];
    __shared__ unsigned long long wbest[kProposeThreads / kWave];
    propose_block(tokens, cap, state, nmax, K, drafts, tk, kChunk, wbest);
}

__global__ __launch_bounds__(kWave) void accept_kernel(const int32_t* __restrict__ argmax,
                                                       const int32_t* __restrict__ drafts, int K,
                                                       int32_t* __restrict__ tokens, int cap,
                                                       int32_t* __restrict__ state) {
    accept_wave(argmax, drafts, K, tokens, cap, state, threadIdx.x);
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
