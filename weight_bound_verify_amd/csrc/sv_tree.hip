// Greedy tree verify ("Stream C - Speculative decoding", EAGLE-3 + tree handoff and the
// deferred list: the drafter proposes a tree, one verify forward covers every node, and the
// linear accept becomes a walk down the tree).
//
// A tree of K <= 15 draft nodes hangs under the anchor (node 0): node i (1..K) has parent
// parents[i-1] < i and token drafts[i-1] (a pad -1 never matches).  The head matmul is the
// linear one over S = K+1 window rows; only the tail differs:
//   accept  from node c = 0, move to the lowest-index child whose token is argmax[c], until
//           none matches; the path's tokens and the last argmax are committed (len += 1 + j);
//   drafter the best `branches` earlier matches of the stream's suffix, ranked as the linear
//           drafter ranks them (longer match, then more recent), each continued for `depth`
//           tokens and merged into a prefix tree in rank order until K nodes exist.
// The drafter runs on one workgroup: every thread keeps the four best (length, end) keys of
// its end positions, four block-wide max reductions take the global best four, and wave 0
// builds the prefix tree with one lane per (branch, depth) slot: a slot opens a node iff no
// earlier branch has the same prefix up to that depth, and node indices are the running count
// of opened slots in (branch, depth) order, which is the insertion order of a sequential trie.
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_tail.h"

#include <climits>
#include <cmath>

namespace sv {

namespace {

constexpr int kTreeThreads = 1024;
constexpr int kTreeIds = 32768;                      // stream ids held in LDS (128 KB)
constexpr int kMaxBranches = 4;

// Walk down the tree by one wave (lane i holds node i+1).  `am` holds the argmax of every
// window row.  Appends the path's tokens and the final argmax to `tokens` (and `mirror` when
// not null), advances len, records the round.  Returns j, or -1 when `cap` would overflow
// (nothing written, capacity flag set).
__device__ __forceinline__ int accept_tree_wave(const int32_t* am, const int32_t* parents, const int32_t* drafts,
                                                int K, int32_t* tokens, int cap, int32_t* state, int lane,
                                                int32_t* mirror, const StateCache* cache = nullptr) {
    const int len = cache ? state_word(*cache, SV_STATE_LEN) : state[SV_STATE_LEN];
    if (len + K + 1 > cap || len < 0) {
        if (lane == 0) state[SV_STATE_FLAGS] |= SV_FLAG_CAPACITY;
        return -1;
    }
    int par = -1, tok = -1;
    if (lane < K) { par = parents[lane]; tok = drafts[lane]; }
    int c = 0, j = 0, pos = -1;
    for (int step = 0; step < K; ++step) {             // a path has at most K nodes
        const int a = am[c];
        // a parent index must precede its node (par <= lane), so the walk only moves forward
        const unsigned long long m = __ballot(lane < K && par == c && par <= lane && tok >= 0 && tok == a);
        if (m == 0) break;
        const int nxt = __builtin_ctzll(m);           // lowest node index
        if (lane == nxt) pos = j;
        c = nxt + 1;
        ++j;
    }
    if (pos >= 0) {
        tokens[len + pos] = tok;
        if (mirror) mirror[len + pos] = tok;
    }
    if (lane == 0) {
        const int fin = am[c];
        tokens[len + j] = fin;
        if (mirror) mirror[len + j] = fin;
        state[SV_STATE_LEN] = len + 1 + j;
        if (!cache) record_round(state, j);
    }
    if (cache) record_round_cached(*cache, state, j, lane);
    return j;
}

// Block-wide maximum of one 64-bit key per thread; every thread gets the result.
__device__ __forceinline__ unsigned long long block_max_u64(unsigned long long v, unsigned long long* wslot,
                                                            unsigned long long* result) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    const int tid = threadIdx.x;
    if ((tid & 63) == 0) wslot[tid >> 6] = v;
    __syncthreads();
    if (tid < kWave) {
        unsigned long long b = tid < (int)(blockDim.x / kWave) ? wslot[tid] : 0ull;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const unsigned long long o = __shfl_xor(b, off, 64);
            b = o > b ? o : b;
        }
        if (tid == 0) *result = b;
    }
    __syncthreads();
    return *result;
}

// Tree drafter over the stream `st[0 .. len)` (LDS or global memory), whole workgroup.
// `keys` (LDS, kMaxBranches + 1 entries) and `wslot` (one per wave) are scratch.
__device__ __forceinline__ void propose_tree_block(const int32_t* st, int len, int nmax, int K, int branches,
                                                   int depth, int32_t* parents_out, int32_t* drafts_out,
                                                   int32_t* state, bool gated, unsigned long long* keys,
                                                   unsigned long long* wslot) {
    const int tid = threadIdx.x;
    if (gated) {
        if (tid < K) { parents_out[tid] = 0; drafts_out[tid] = -1; }
        if (tid == 0) { state[SV_STATE_NVALID] = 0; state[SV_STATE_NUSED] = 0; }
        return;
    }
    int32_t suf[SV_MAX_NGRAM];
#pragma unroll
    for (int i = 0; i < SV_MAX_NGRAM; ++i) suf[i] = (i < nmax && len - 1 - i >= 0) ? st[len - 1 - i] : -1;
    // the four best keys (l << 32 | e) of this thread's end positions, best first
    unsigned long long top[kMaxBranches] = {0ull, 0ull, 0ull, 0ull};
    for (int e = tid; e < len - 1; e += blockDim.x) {
        int l = 0;
#pragma unroll
        for (int i = 0; i < SV_MAX_NGRAM; ++i)
            if (l == i && i < nmax && e - i >= 0 && st[e - i] == suf[i]) l = i + 1;
        if (l > 0) {
            unsigned long long k = ((unsigned long long)l << 32) | (unsigned)e;
#pragma unroll
            for (int b = 0; b < kMaxBranches; ++b) {       // sorted insertion
                if (k > top[b]) { const unsigned long long t = top[b]; top[b] = k; k = t; }
            }
        }
    }
    // the global best `branches` keys: each round takes the largest key below the previous one
    unsigned long long thr = ~0ull;
    for (int b = 0; b < branches; ++b) {
        unsigned long long mine = 0ull;
#pragma unroll
        for (int t = kMaxBranches - 1; t >= 0; --t)
            if (top[t] < thr && top[t] > mine) mine = top[t];
        const unsigned long long best = block_max_u64(mine, wslot, &keys[kMaxBranches]);
        if (tid == 0) keys[b] = best;
        thr = best;
        if (best == 0ull) {                             // no further match (uniform)
            if (tid == 0)
                for (int r = b + 1; r < branches; ++r) keys[r] = 0ull;
            break;
        }
    }
    __syncthreads();
    if (tid >= kWave) return;
    // wave 0: lane = branch * 16 + depth slot
    const int lane = tid;
    const int b = lane >> 4, d = lane & 15;
    int e[kMaxBranches], clen[kMaxBranches];
#pragma unroll
    for (int r = 0; r < kMaxBranches; ++r) {
        const unsigned long long k = r < branches ? keys[r] : 0ull;
        e[r] = (int)(k & 0xffffffffu);
        const int avail = len - 1 - e[r];
        clen[r] = k == 0ull ? 0 : (avail < depth ? avail : depth);
    }
    int eb = 0, cb = 0;
#pragma unroll
    for (int r = 0; r < kMaxBranches; ++r)
        if (r == b) { eb = e[r]; cb = clen[r]; }
    const bool active = d < cb;
    const int tok = active ? st[eb + 1 + d] : -1;
    // first branch with the same prefix of length d + 1
    int first = b;
    if (active) {
#pragma unroll
        for (int r = 0; r < kMaxBranches; ++r) {
            if (r < b && first == b && d < clen[r]) {
                bool same = true;
                for (int k = 0; k <= d && same; ++k) same = st[e[r] + 1 + k] == st[eb + 1 + k];
                if (same) first = r;
            }
        }
    }
    const bool opens = active && first == b;
    const unsigned long long om = __ballot(opens);
    const int own = 1 + __popcll(om & ((1ull << lane) - 1ull));
    const int src = active ? first * 16 + d : lane;
    const int idx = __shfl(own, src, 64);               // node of this slot's prefix
    const int pidx_src = d > 0 ? lane - 1 : lane;
    const int pidx_raw = __shfl(idx, pidx_src, 64);
    const int pidx = d > 0 ? pidx_raw : 0;
    if (opens && idx <= K) {
        parents_out[idx - 1] = pidx;
        drafts_out[idx - 1] = tok;
    }
    const int opened = __popcll(om);
    const int real = opened < K ? opened : K;
    if (lane >= real && lane < K) { parents_out[lane] = 0; drafts_out[lane] = -1; }
    if (lane == 0) {
        state[SV_STATE_NVALID] = real;
        state[SV_STATE_NUSED] = keys[0] == 0ull ? 0 : (int)(keys[0] >> 32);
    }
}

// Argmax stage 2 of one window row: fold the per-workgroup partials in a fixed order.
__device__ __forceinline__ int reduce_argmax_row(const float* __restrict__ pv, const int* __restrict__ pi,
                                                 int nparts, int s, int lane) {
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int p0 = 0; p0 < nparts; p0 += 8 * kWave) {
        float v[8];
        int ix[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = p0 + u * kWave + lane;
            v[u] = p < nparts ? pv[(size_t)s * kGridMax + p] : -INFINITY;
            ix[u] = p < nparts ? pi[(size_t)s * kGridMax + p] : INT_MAX;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (better(v[u], ix[u], bv, bi)) { bv = v[u]; bi = ix[u]; }
    }
    argmax_group<64>(bv, bi);
    return bi;
}

// Tree round tail: argmax of every node row, the walk, the next tree.  One workgroup.
__global__ __launch_bounds__(kTreeThreads) void tree_tail_kernel(
    const float* __restrict__ pv, const int* __restrict__ pi, int nparts, int S, int32_t* __restrict__ argmax,
    const int32_t* __restrict__ parents_in, const int32_t* __restrict__ drafts_in, int32_t* __restrict__ tokens,
    int cap, int32_t* __restrict__ state, int nmax, int branches, int depth, int32_t* __restrict__ parents_out,
    int32_t* __restrict__ drafts_out) {
    __shared__ __attribute__((aligned(16))) int32_t tk[kTreeIds];
    __shared__ int32_t am[16];
    __shared__ int new_len;
    __shared__ int gated_s;
    __shared__ unsigned long long keys[kMaxBranches + 1];
    __shared__ unsigned long long wslot[kTreeThreads / kWave];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int K = S - 1;
    const int len0 = state[SV_STATE_LEN];
    StateCache sc{0, 0};
    if (wave == 0) sc = state_cache_load(state, lane);
    const bool in_lds = len0 >= 0 && len0 + K + 1 <= cap && len0 + K + 1 <= kTreeIds;
    if (in_lds) stage_ids(tokens, len0, tk);
    for (int s = wave; s < S; s += kTreeThreads / kWave) {
        const int bi = reduce_argmax_row(pv, pi, nparts, s, lane);
        if (lane == 0) { argmax[s] = bi; am[s] = bi; }
    }
    __syncthreads();
    if (wave == 0) {
        const int j = accept_tree_wave(am, parents_in, drafts_in, K, tokens, cap, state, lane, in_lds ? tk : nullptr,
                                       &sc);
        // the gate word after this round, as the walk recorded it (no round recorded when j < 0)
        const int zero_run = j == 0 ? state_word(sc, SV_STATE_ZERO_RUN) + 1 : 0;
        const int gate_after = state_word(sc, SV_STATE_GATE_AFTER);
        const bool gated = state_word(sc, SV_STATE_GATED) != 0 || (j >= 0 && gate_after > 0 && zero_run >= gate_after);
        if (lane == 0) {
            new_len = j >= 0 ? len0 + 1 + j : len0;
            gated_s = gated;
        }
    }
    __syncthreads();
    int len = new_len;
    const int32_t* st = tk;
    if (!in_lds) {                                     // long or corrupt stream: global memory
        st = tokens;
        if (len < 0 || len > cap) {
            if (threadIdx.x == 0) state[SV_STATE_FLAGS] |= SV_FLAG_CAPACITY;
            len = 0;
        }
    }
    propose_tree_block(st, len, nmax, K, branches, depth, parents_out, drafts_out, state, gated_s != 0, keys, wslot);
}

__global__ __launch_bounds__(kTreeThreads) void propose_tree_kernel(const int32_t* __restrict__ tokens, int cap,
                                                                   int32_t* __restrict__ state, int nmax, int K,
                                                                   int branches, int depth,
                                                                   int32_t* __restrict__ parents_out,
                                                                   int32_t* __restrict__ drafts_out) {
    __shared__ __attribute__((aligned(16))) int32_t tk[kTreeIds];
    __shared__ unsigned long long keys[kMaxBranches + 1];
    __shared__ unsigned long long wslot[kTreeThreads / kWave];
    int len = state[SV_STATE_LEN];
    const bool gated = state[SV_STATE_GATED] != 0;
    if (len < 0 || len > cap) {
        if (threadIdx.x == 0) state[SV_STATE_FLAGS] |= SV_FLAG_CAPACITY;
        len = 0;
    }
    const int32_t* st = tokens;
    if (len <= kTreeIds) {
        stage_ids(tokens, len, tk);
        __syncthreads();
        st = tk;
    }
    propose_tree_block(st, len, nmax, K, branches, depth, parents_out, drafts_out, state, gated, keys, wslot);
}

__global__ __launch_bounds__(kWave) void accept_tree_kernel(const int32_t* __restrict__ argmax,
                                                            const int32_t* __restrict__ parents,
                                                            const int32_t* __restrict__ drafts, int K,
                                                            int32_t* __restrict__ tokens, int cap,
                                                            int32_t* __restrict__ state) {
    __shared__ int32_t am[16];
    if (threadIdx.x <= K) am[threadIdx.x] = argmax[threadIdx.x];
    __syncthreads();
    accept_tree_wave(am, parents, drafts, K, tokens, cap, state, threadIdx.x, nullptr);
}

}  // namespace

hipError_t launch_tree_tail(const float* pv, const int* pi, int nparts, int S, int32_t* argmax,
                            const int32_t* parents_in, const int32_t* drafts_in, int32_t* tokens, int cap,
                            int32_t* state, int nmax, int branches, int depth, int32_t* parents_out,
                            int32_t* drafts_out, hipStream_t stream) {
    hipLaunchKernelGGL(tree_tail_kernel, dim3(1), dim3(kTreeThreads), 0, stream, pv, pi, nparts, S, argmax,
                       parents_in, drafts_in, tokens, cap, state, nmax, branches, depth, parents_out, drafts_out);
    return hipGetLastError();
}

hipError_t launch_propose_tree(const int32_t* tokens, int cap, int32_t* state, int nmax, int K, int branches,
                               int depth, int32_t* parents_out, int32_t* drafts_out, hipStream_t stream) {
    hipLaunchKernelGGL(propose_tree_kernel, dim3(1), dim3(kTreeThreads), 0, stream, tokens, cap, state, nmax, K,
                       branches, depth, parents_out, drafts_out);
    return hipGetLastError();
}

hipError_t launch_accept_tree(const int32_t* argmax, const int32_t* parents, const int32_t* drafts, int K,
                              int32_t* tokens, int cap, int32_t* state, hipStream_t stream) {
    hipLaunchKernelGGL(accept_tree_kernel, dim3(1), dim3(kWave), 0, stream, argmax, parents, drafts, K, tokens, cap,
                       state);
    return hipGetLastError();
}

}  // namespace sv
