// Row kernels of the dense stack: the weightless RMSNorm and the combine of a split down
// projection fused with the residual add and the next block's RMSNorm.
//
// Page: "Flagship dramatic-speedup plan - the full stackable tuning set", section "Axis 4"
// (RMSNorm fused into the neighbouring kernels).  The pages leave the norm itself open; the
// library reads it as the weightless pre-norm n = fp16(x / sqrt(mean(x^2) + eps)), with the
// sum of squares in fp32 over the fp16 values of x.
//
// One workgroup per window row.  Each thread owns the columns tid + j*kRowThreads
// (j < kRowPer) of every 4096-column pass, issues all loads of a pass before using any of
// them (the data is a few hundred KB, so the kernel is bound by memory latency, not bytes),
// and keeps the row in registers when it fits in one pass.  The reduction order is fixed.
#include "sv_device.h"
#include "sv_internal.h"

namespace sv {

namespace {

constexpr int kRowThreads = 1024;
constexpr int kRowPer = 4;
constexpr int kRowPass = kRowThreads * kRowPer;
constexpr int kMaxSplit = kRowNormMaxSplit;

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kRowThreads / kWave; ++w) t += red[w];
    return t;
}

// For window row s:
//   t[n] = sum_{k < ks} part[k][s][n] (+ residual[s][n])       (ks = 0: t = residual)
//   y[s][n] = fp16(t[n])                                        (skipped when y is null)
//   norm_out[s][n] = fp16(fp16(t[n]) / sqrt(mean_n fp16(t[n])^2 + eps))
// y may alias residual, and norm_out may alias residual when y is null: every element is
// read before it is written, by the thread that writes it.
__global__ __launch_bounds__(kRowThreads) void row_norm_kernel(const float* __restrict__ part, int ks, int S, int N,
                                                               const uint16_t* residual, uint16_t* y, float eps,
                                                               uint16_t* norm_out) {
    __shared__ float red[kRowThreads / kWave];
    const int tid = threadIdx.x;
    const size_t row = (size_t)blockIdx.x * N;
    const size_t plane = (size_t)S * N;
    float keep[kRowPer];
    float ss = 0.f;
    for (int base = 0; base < N; base += kRowPass) {
        float p[kRowPer][kMaxSplit];
        float r[kRowPer];
#pragma unroll
        for (int j = 0; j < kRowPer; ++j) {
            const int v = base + j * kRowThreads + tid;
#pragma unroll
            for (int k = 0; k < kMaxSplit; ++k) p[j][k] = (k < ks && v < N) ? part[k * plane + row + v] : 0.f;
            r[j] = (residual && v < N) ? h2f(residual[row + v]) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kRowPer; ++j) {
            const int v = base + j * kRowThreads + tid;
            float t = p[j][0];
#pragma unroll
            for (int k = 1; k < kMaxSplit; ++k) if (k < ks) t += p[j][k];
            t = ks > 0 ? t + r[j] : r[j];
            const uint16_t h = f2h(t);
            const float q = h2f(h);
            keep[j] = q;
            if (v < N) {
                if (y) y[row + v] = h;
                ss = __builtin_fmaf(q, q, ss);
            }
        }
    }
    const float inv = 1.0f / sqrtf(block_sum(ss, red) / (float)N + eps);
    const uint16_t* again = y ? y : residual;     // rows longer than one pass are re-read
    for (int base = 0; base < N; base += kRowPass) {
#pragma unroll
        for (int j = 0; j < kRowPer; ++j) {
            const int v = base + j * kRowThreads + tid;
            if (v < N) {
                const float q = N <= kRowPass ? keep[j] : h2f(again[row + v]);
                norm_out[row + v] = f2h(q * inv);
            }
        }
    }
}

}  // namespace

hipError_t launch_row_norm(const float* part, int ks, int S, int N, const uint16_t* residual, uint16_t* y,
                           float eps, uint16_t* norm_out, hipStream_t stream) {
    if (ks < 0 || ks > kMaxSplit) return hipErrorInvalidValue;
    hipLaunchKernelGGL(row_norm_kernel, dim3(S), dim3(kRowThreads), 0, stream, part, ks, S, N, residual, y, eps,
                       norm_out);
    return hipGetLastError();
}

}  // namespace sv
