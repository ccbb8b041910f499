// Standalone round kernels around the head matmul: n-gram drafter and greedy accept.
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

}  // namespace sv
