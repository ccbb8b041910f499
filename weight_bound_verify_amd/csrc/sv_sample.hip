// Sampling verify, stage 2 ("Stream C - Speculative decoding", the deferred list: lossless
// sampling at temperature > 0 verifies with probabilities and redraws a rejected position from
// the residual distribution).
//
// The head matmul's sampling epilogue leaves, per window row s and workgroup, the best
// Gumbel key z + g over the row's ids with the row's draft left out (z = L / T, g the Gumbel
// noise of (row, id)), its id, and the row's running (max z, sum exp(z - max)).  With a
// point-mass drafter this is all speculative sampling needs:
//   the row's draw from the residual max(0, p_s - e_d) is the argmax of the keys (Gumbel-max
//   over the ids other than d, whose law is p_s renormalised without d);
//   p_s(d) = exp(z_d - lse_s) decides whether d is kept.
// The tail reduces the partials in a fixed order, then (for a round) accepts from the first
// draft on and drafts the next round, exactly as the greedy tail does.
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_tail.h"

#include <climits>
#include <cmath>

namespace sv {

namespace {

constexpr int kTailThreads = 1024;
constexpr int kTailIds = 32768;                      // stream ids the tail can hold in LDS (128 KB)

// Reduce row s's partials: the best (key, id), lowest id on equal keys, and the merged
// log-sum-exp state.  Each lane folds its partials in increasing order, then the wave folds
// the lanes with a fixed butterfly; lane 0 returns the row's draw and log-normaliser.
__device__ __forceinline__ void reduce_row(const float* __restrict__ pv, const int* __restrict__ pi,
                                           const float* __restrict__ pm, const float* __restrict__ pl, int nparts,
                                           int s, int lane, int& draw, float& lse) {
    float bv = -INFINITY, m = -INFINITY, l = 0.0f;
    int bi = INT_MAX;
    for (int p0 = 0; p0 < nparts; p0 += 4 * kWave) {              // 4 partials in flight per lane
        float v[4], mm[4], ll[4];
        int ix[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = p0 + u * kWave + lane;
            const bool ok = p < nparts;
            const size_t o = (size_t)s * kGridMax + p;
            v[u] = ok ? pv[o] : -INFINITY;
            ix[u] = ok ? pi[o] : INT_MAX;
            mm[u] = ok ? pm[o] : -INFINITY;
            ll[u] = ok ? pl[o] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (better(v[u], ix[u], bv, bi)) { bv = v[u]; bi = ix[u]; }
            lse_merge(m, l, mm[u], ll[u]);
        }
    }
    argmax_group<64>(bv, bi);
    lse_merge_group<64>(m, l);
    draw = bi == INT_MAX ? -1 : bi;                  // -1: every id of the row was left out
    lse = m + __logf(l);
}

__global__ __launch_bounds__(kTailThreads) void sample_tail_kernel(
    const float* __restrict__ pv, const int* __restrict__ pi, const float* __restrict__ pm,
    const float* __restrict__ pl, int nparts, int S, int V, const float* __restrict__ zd, uint32_t key0,
    uint32_t key1, int32_t* __restrict__ sample_out, float* __restrict__ lse_out,
    const int32_t* __restrict__ drafts_in, int32_t* __restrict__ tokens, int cap, int32_t* __restrict__ state,
    int nmax, int32_t* __restrict__ drafts_out) {
    __shared__ __attribute__((aligned(16))) int32_t tk[kTailIds + 8];    // + group reads past the end
    __shared__ int32_t draw_s[16];
    __shared__ float lse_s[16];
    __shared__ int new_len;
    __shared__ int gated_s;
    __shared__ unsigned long long wbest[kTailThreads / kWave];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int K = S - 1;
    const bool round = tokens != nullptr;

    // the stream's first min(cap, kTailIds) ids are loaded with the partials, whatever its length
    int len0 = 0;
    bool in_lds = false;
    IdPrefix<kTailIds / (4 * kTailThreads)> pre;
    const int navail = round ? (cap < kTailIds ? cap : kTailIds) : 0;
    const bool vec = round && (reinterpret_cast<uintptr_t>(tokens) & 15) == 0;
    if (vec) prefix_load(tokens, navail, pre);
    StateCache sc{0, 0};
    int d0 = -1;                                       // wave 0: the round's drafts and their scaled logits
    float zd0 = 0.f;
    if (round) {
        len0 = state[SV_STATE_LEN];
        if (wave == 0) {
            sc = state_cache_load(state, lane);
            if (lane < K) {
                d0 = drafts_in[lane];
                zd0 = zd[lane];
            }
        }
        in_lds = len0 >= 0 && len0 + K + 1 <= cap && len0 + K + 1 <= kTailIds;
    }
    for (int s = wave; s < S; s += kTailThreads / kWave) {
        int draw;
        float lse;
        reduce_row(pv, pi, pm, pl, nparts, s, lane, draw, lse);
        if (lane == 0) {
            draw_s[s] = draw;
            lse_s[s] = lse;
            if (sample_out) sample_out[s] = draw;
            if (lse_out) lse_out[s] = lse;
        }
    }
    if (!round) return;
    if (in_lds) {
        if (vec) prefix_store(tokens, navail, pre, tk);
        else stage_ids(tokens, len0, tk);
    }
    if (!in_lds) {                                     // long or corrupt stream: the global-memory path
        __syncthreads();
        if (wave == 0) accept_sample_regs(draw_s, lse_s, d0, zd0, K, V, key0, key1, tokens, cap, state, lane, nullptr);
        __syncthreads();
        propose_block(tokens, cap, state, nmax, K, drafts_out, tk, kTailIds - kHalo, wbest);
        return;
    }
    barrier_lds();                                     // the stream and the draws are in LDS
    if (wave == 0) {
        const int j = accept_sample_regs(draw_s, lse_s, d0, zd0, K, V, key0, key1, tokens, cap, state, lane, tk, &sc);
        // the gate word after this round: recomputed from the cache as the accept recorded it
        const int zero_run = j == 0 ? state_word(sc, SV_STATE_ZERO_RUN) + 1 : 0;
        const int gate_after = state_word(sc, SV_STATE_GATE_AFTER);
        const bool gated = state_word(sc, SV_STATE_GATED) != 0 || (K > 0 && gate_after > 0 && zero_run >= gate_after);
        if (lane == 0) {
            new_len = len0 + 1 + j;
            gated_s = gated;
        }
    }
    barrier_lds();                                     // the drafter reads only LDS (tk, new_len, gated_s)
    propose_lds(tk, new_len, nmax, K, drafts_out, state, wbest, gated_s != 0);
}

__global__ __launch_bounds__(kWave) void accept_sample_kernel(const int32_t* __restrict__ sample,
                                                              const float* __restrict__ lse,
                                                              const float* __restrict__ zd,
                                                              const int32_t* __restrict__ drafts, int K, int V,
                                                              uint32_t key0, uint32_t key1,
                                                              int32_t* __restrict__ tokens, int cap,
                                                              int32_t* __restrict__ state) {
    accept_sample_wave(sample, lse, zd, drafts, K, V, key0, key1, tokens, cap, state, threadIdx.x, nullptr);
}

}  // namespace

hipError_t launch_sample_tail(const float* pv, const int* pi, const float* pm, const float* pl, int nparts, int S,
                              int V, const float* zd, uint32_t key0, uint32_t key1, int32_t* sample_out,
                              float* lse_out, const int32_t* drafts_in, int32_t* tokens, int cap, int32_t* state,
                              int nmax, int32_t* drafts_out, hipStream_t stream) {
    hipLaunchKernelGGL(sample_tail_kernel, dim3(1), dim3(kTailThreads), 0, stream, pv, pi, pm, pl, nparts, S, V, zd,
                       key0, key1, sample_out, lse_out, drafts_in, tokens, cap, state, nmax, drafts_out);
    return hipGetLastError();
}

hipError_t launch_accept_sample(const int32_t* sample, const float* lse, const float* zd, const int32_t* drafts,
                                int K, int V, uint32_t key0, uint32_t key1, int32_t* tokens, int cap,
                                int32_t* state, hipStream_t stream) {
    hipLaunchKernelGGL(accept_sample_kernel, dim3(1), dim3(kWave), 0, stream, sample, lse, zd, drafts, K, V, key0,
                       key1, tokens, cap, state);
    return hipGetLastError();
}

}  // namespace sv
