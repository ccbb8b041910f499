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
    __shared__ __attribute__((aligned(16))) int32_t tk[kHalo + kChunk];
    __shared__ unsigned long long wbest[kProposeThreads / kWave];
    propose_block(tokens, cap, state, nmax, K, drafts, tk, kChunk, wbest);
}

__global__ __launch_bounds__(kWave) void accept_kernel(const int32_t* __restrict__ argmax,
                                                       const int32_t* __restrict__ drafts, int K,
                                                       int32_t* __restrict__ tokens, int cap,
                                                       int32_t* __restrict__ state) {
    accept_wave(argmax, drafts, K, tokens, cap, state, threadIdx.x);
}

// Window rows of a token-indexed stand-in model: row 0 = table[tokens[len-1]] (the anchor),
// row i = table[drafts[i-1]] with a pad (-1) reading token 0's row.  One workgroup per row,
// 16-byte copies.  An id outside [0, V) writes a zero row and sets the token flag; a length
// outside [1, cap] writes zero rows and sets the capacity flag.
__global__ __launch_bounds__(256) void gather_window_kernel(const int32_t* __restrict__ tokens, int cap,
                                                            int32_t* __restrict__ state,
                                                            const int32_t* __restrict__ drafts,
                                                            const uint16_t* __restrict__ table, int V, int H,
                                                            uint16_t* __restrict__ out) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const int r = blockIdx.x;
    const int len = state[SV_STATE_LEN];
    const bool len_ok = len >= 1 && len <= cap;
    int id;
    if (r == 0) id = len_ok ? tokens[len - 1] : -1;
    else id = drafts[r - 1] >= 0 ? drafts[r - 1] : 0;
    const bool ok = len_ok && id >= 0 && id < V;
    if (threadIdx.x == 0 && !ok) atomicOr(&state[SV_STATE_FLAGS], len_ok ? SV_FLAG_TOKEN : SV_FLAG_CAPACITY);
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(table + (size_t)(ok ? id : 0) * H);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + (size_t)r * H);
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    for (int i = threadIdx.x; i < H / 8; i += 256) dst[i] = ok ? src[i] : zero;
}

// Window rows of a position-indexed stand-in model: row i = rows[len - 1 + i] (the row after a
// prefix of len + i ids), one workgroup per row, 16-byte copies.  A position outside
// [0, nrows) or a length outside [1, cap] writes a zero row and sets the capacity flag.
__global__ __launch_bounds__(256) void gather_positions_kernel(int32_t* __restrict__ state, int cap,
                                                               const uint16_t* __restrict__ rows, int nrows, int H,
                                                               uint16_t* __restrict__ out) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const int r = blockIdx.x;
    const int len = state[SV_STATE_LEN];
    const long long p = (long long)len - 1 + r;
    const bool ok = len >= 1 && len <= cap && p >= 0 && p < nrows;
    if (threadIdx.x == 0 && !ok) atomicOr(&state[SV_STATE_FLAGS], SV_FLAG_CAPACITY);
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(rows + (size_t)(ok ? p : 0) * H);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + (size_t)r * H);
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    for (int i = threadIdx.x; i < H / 8; i += 256) dst[i] = ok ? src[i] : zero;
}

}  // namespace

hipError_t launch_gather_positions(int32_t* state, int cap, const uint16_t* rows, int nrows, int H, int S,
                                   uint16_t* out, hipStream_t stream) {
    hipLaunchKernelGGL(gather_positions_kernel, dim3(S), dim3(256), 0, stream, state, cap, rows, nrows, H, out);
    return hipGetLastError();
}

hipError_t launch_gather_window(const int32_t* tokens, int cap, int32_t* state, const int32_t* drafts, int K,
                                const uint16_t* table, int V, int H, uint16_t* out, hipStream_t stream) {
    hipLaunchKernelGGL(gather_window_kernel, dim3(K + 1), dim3(256), 0, stream, tokens, cap, state, drafts, table, V,
                       H, out);
    return hipGetLastError();
}

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
