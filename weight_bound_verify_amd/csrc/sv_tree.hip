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
constexpr int kTreeHead = 8192;                      // stream ids loaded before the length is known

// Walk down the tree by one wave, the tree in registers: lane i < K holds node i+1 (its parent
// `par`, its token `tok`; -1 on the other lanes).  `am` holds the argmax of every window row.
// Appends the path's tokens and the final argmax to `tokens` (and `mirror` when not null),
// advances len, records the round.  Returns j, or -1 when `cap` would overflow (nothing
// written, capacity flag set).
__device__ __forceinline__ int accept_tree_regs(const int32_t* am, int par, int tok, int K, int32_t* tokens, int cap,
                                                int32_t* state, int lane, int32_t* mirror,
                                                const StateCache* cache = nullptr) {
    const int len = cache ? state_word(*cache, SV_STATE_LEN) : state[SV_STATE_LEN];
    if (len + K + 1 > cap || len < 0) {
        if (lane == 0) state[SV_STATE_FLAGS] |= SV_FLAG_CAPACITY;
        return -1;
    }
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
    const int fin = am[c];                             // the correction or bonus id (uniform)
    if (fin < 0) {                                     // that row had no greedy id: commit nothing
        if (lane == 0) state[SV_STATE_FLAGS] |= SV_FLAG_ARGMAX;
        return -1;
    }
    if (pos >= 0) {
        tokens[len + pos] = tok;
        if (mirror) mirror[len + pos] = tok;
    }
    if (lane == 0) {
        tokens[len + j] = fin;
        if (mirror) mirror[len + j] = fin;
        state[SV_STATE_LEN] = len + 1 + j;
        if (!cache) record_round(state, j);
    }
    if (cache) record_round_cached(*cache, state, j, lane);
    return j;
}

// The same walk with the tree read from `parents` / `drafts` (K entries each).
__device__ __forceinline__ int accept_tree_wave(const int32_t* am, const int32_t* parents, const int32_t* drafts,
                                                int K, int32_t* tokens, int cap, int32_t* state, int lane,
                                                int32_t* mirror) {
    int par = -1, tok = -1;
    if (lane < K) { par = parents[lane]; tok = drafts[lane]; }
    return accept_tree_regs(am, par, tok, K, tokens, cap, state, lane, mirror);
}

// The same over a stream in global memory, one end position per thread and step.
__device__ __forceinline__ void scan_top_global(const int32_t* st, int len, int nmax,
                                                const int32_t (&suf)[SV_MAX_NGRAM],
                                                unsigned long long (&top)[kMaxBranches]) {
    for (int e = threadIdx.x; e < len - 1; e += blockDim.x) {
        int l = 0;
#pragma unroll
        for (int i = 0; i < SV_MAX_NGRAM; ++i)
            if (l == i && i < nmax && e - i >= 0 && st[e - i] == suf[i]) l = i + 1;
        if (l > 0) top_insert(top, ((unsigned long long)l << 32) | (unsigned)e);
    }
}

// The best `branches` of 64 candidate keys (one per lane; distinct or zero), in order, by
// `branches` wave maxima each below the previous one; every lane gets them.
// (match length, end position) keys of streams shorter than 2^27 ids fit 32 bits, l << 27 | e,
// in the same order as l << 32 | e; their wave maxima then take DPP moves instead of 64-bit
// shuffles (measured in the c3tree round's tail: the two merges took 3.3 of its 9.4 us).
constexpr int kKeyShift32 = 27;
__device__ __forceinline__ uint32_t key_narrow(unsigned long long k) {
    return (uint32_t)(((k >> 32) << kKeyShift32) | (k & 0xffffffffull));
}
__device__ __forceinline__ unsigned long long key_wide(uint32_t k) {
    return ((unsigned long long)(k >> kKeyShift32) << 32) | (k & ((1u << kKeyShift32) - 1u));
}

// wave_top over narrow keys; all 64 lanes active
__device__ __forceinline__ void wave_top32(uint32_t cand, int branches, unsigned long long (&out)[kMaxBranches]) {
    uint32_t thr = ~0u;
#pragma unroll
    for (int b = 0; b < kMaxBranches; ++b) {
        const uint32_t v = wave_max_u32(b < branches && cand < thr ? cand : 0u);
        out[b] = b < branches ? key_wide(v) : 0ull;
        thr = v;
    }
}

__device__ __forceinline__ void wave_top(unsigned long long cand, int branches, unsigned long long (&out)[kMaxBranches]) {
    unsigned long long thr = ~0ull;
#pragma unroll
    for (int b = 0; b < kMaxBranches; ++b) {
        unsigned long long v = b < branches && cand < thr ? cand : 0ull;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const unsigned long long o = __shfl_xor(v, off, 64);
            v = o > v ? o : v;
        }
        out[b] = b < branches ? v : 0ull;
        thr = v;
    }
}

// Tree drafter over the stream `st[0 .. len)` (LDS when `in_lds`, else global memory), whole
// workgroup.  `keys` (LDS, kMaxBranches + 1 entries) and `wkeys` (kMaxBranches per wave) are
// scratch.
__device__ __forceinline__ void propose_tree_block(const int32_t* st, bool in_lds, int len, int nmax, int K,
                                                   int branches, int depth, int32_t* parents_out,
                                                   int32_t* drafts_out, int32_t* state, bool gated,
                                                   unsigned long long* keys, unsigned long long* wkeys) {
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
    if (in_lds) {
        if (nmax <= 4) scan_top_lds<4>(st, len, nmax, suf, top, threadIdx.x, blockDim.x);
        else scan_top_lds<8>(st, len, nmax, suf, top, threadIdx.x, blockDim.x);
    } else {
        scan_top_global(st, len, nmax, suf, top);
    }
    // the global best `branches` keys: the wave's best from its lanes' lists (the best b of a
    // set lie among the best b of every part), one barrier, then wave 0 over the waves' lists
    const int lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x / kWave;
    unsigned long long wbest[kMaxBranches];
    const bool narrow = len < (1 << kKeyShift32);     // uniform: every key fits 32 bits
    if (narrow) {
        // the same selection as below on 32-bit keys
        uint32_t t32[kMaxBranches];
#pragma unroll
        for (int r = 0; r < kMaxBranches; ++r) t32[r] = key_narrow(top[r]);
        uint32_t thr = ~0u;
#pragma unroll
        for (int b = 0; b < kMaxBranches; ++b) {
            uint32_t mine = 0u;
#pragma unroll
            for (int r = 0; r < kMaxBranches; ++r)
                if (t32[r] < thr && t32[r] > mine) mine = t32[r];
            const uint32_t v = wave_max_u32(b < branches ? mine : 0u);
            wbest[b] = key_wide(v);
            thr = v;
        }
    } else {
        // lane candidates: its own list, merged round by round below the previous maximum
        unsigned long long thr = ~0ull;
#pragma unroll
        for (int b = 0; b < kMaxBranches; ++b) {
            unsigned long long mine = 0ull;
#pragma unroll
            for (int r = 0; r < kMaxBranches; ++r)
                if (top[r] < thr && top[r] > mine) mine = top[r];
            unsigned long long v = b < branches ? mine : 0ull;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const unsigned long long o = __shfl_xor(v, off, 64);
                v = o > v ? o : v;
            }
            wbest[b] = v;
            thr = v;
        }
    }
    if (lane < kMaxBranches) {
        unsigned long long v = 0ull;
#pragma unroll
        for (int b = 0; b < kMaxBranches; ++b)
            if (b == lane) v = wbest[b];
        wkeys[wave * kMaxBranches + lane] = v;
    }
    __syncthreads();
    if (tid < kWave) {
        const unsigned long long cand = tid < nwaves * kMaxBranches ? wkeys[tid] : 0ull;
        unsigned long long best[kMaxBranches];
        if (narrow) wave_top32(key_narrow(cand), branches, best);
        else wave_top(cand, branches, best);
        if (tid == 0)
#pragma unroll
            for (int b = 0; b < kMaxBranches; ++b) keys[b] = best[b];
    }
    __syncthreads();
    if (tid >= kWave) return;
    // wave 0: lane = branch * 16 + depth slot
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
    __shared__ __attribute__((aligned(16))) int32_t tk[kTreeIds + 8];    // + group reads past the end
    __shared__ int32_t am[16];
    __shared__ int new_len;
    __shared__ int gated_s;
    __shared__ unsigned long long keys[kMaxBranches + 1];
    __shared__ unsigned long long wkeys[kMaxBranches * (kTreeThreads / kWave)];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int K = S - 1;
    // every independent load first: the stream's first min(cap, kTreeHead) ids (whatever its
    // length), the state and the partials; the rest of the stream is loaded once its length is
    // known, only up to it, and the stream goes to LDS once the partials are reduced
    IdPrefix<kTreeHead / (4 * kTreeThreads)> pre;
    IdPrefix<(kTreeIds - kTreeHead) / (4 * kTreeThreads)> pre2;
    const int navail = cap < kTreeIds ? cap : kTreeIds;
    const int nhead = navail < kTreeHead ? navail : kTreeHead;
    const bool vec = (reinterpret_cast<uintptr_t>(tokens) & 15) == 0;
    if (vec) prefix_load(tokens, nhead, pre);
    const int len0 = state[SV_STATE_LEN];
    StateCache sc{0, 0};
    int par0 = -1, tok0 = -1;                          // wave 0: the tree of this round (node lane + 1)
    if (wave == 0) {
        sc = state_cache_load(state, lane);
        if (lane < K) { par0 = parents_in[lane]; tok0 = drafts_in[lane]; }
    }
    const bool in_lds = len0 >= 0 && len0 + K + 1 <= cap && len0 + K + 1 <= kTreeIds;
    for (int s = wave; s < S; s += kTreeThreads / kWave) {
        const int bi = argmax_id(reduce_argmax_row(pv, pi, nparts, s, lane));
        if (lane == 0) { argmax[s] = bi; am[s] = bi; }
    }
    // the stream beyond its first kTreeHead ids, up to its length
    const int nrest = in_lds && len0 > kTreeHead ? len0 : kTreeHead;
    if (vec) prefix_load_from(tokens, kTreeHead, nrest, pre2);
    if (in_lds) {
        if (vec) {
            prefix_store(tokens, nhead < len0 ? nhead : len0, pre, tk);
            prefix_store_from(tokens, kTreeHead, nrest, pre2, tk);
            for (int i = ((len0 >> 2) << 2) + threadIdx.x; i < len0; i += kTreeThreads)    // the ragged end
                if (i >= kTreeHead) tk[i] = tokens[i];
        } else {
            stage_ids(tokens, len0, tk);
        }
    }
    barrier_lds();                                     // the stream (when it fits) and the argmax are in LDS
    if (wave == 0) {
        const int j = accept_tree_regs(am, par0, tok0, K, tokens, cap, state, lane, in_lds ? tk : nullptr, &sc);
        // the gate word after this round, as the walk recorded it (no round recorded when j < 0)
        const int zero_run = j == 0 ? state_word(sc, SV_STATE_ZERO_RUN) + 1 : 0;
        const int gate_after = state_word(sc, SV_STATE_GATE_AFTER);
        const bool gated = state_word(sc, SV_STATE_GATED) != 0 || (j >= 0 && gate_after > 0 && zero_run >= gate_after);
        if (lane == 0) {
            new_len = j >= 0 ? len0 + 1 + j : len0;
            gated_s = gated;
        }
    }
    // the LDS drafter reads only LDS; the global-memory one reads the stream and state just written
    if (in_lds) barrier_lds();
    else __syncthreads();
    int len = new_len;
    const int32_t* st = tk;
    if (!in_lds) {                                     // long or corrupt stream: global memory
        st = tokens;
        if (len < 0 || len > cap) {
            if (threadIdx.x == 0) state[SV_STATE_FLAGS] |= SV_FLAG_CAPACITY;
            len = 0;
        }
    }
    propose_tree_block(st, in_lds, len, nmax, K, branches, depth, parents_out, drafts_out, state, gated_s != 0, keys,
                       wkeys);
}

__global__ __launch_bounds__(kTreeThreads) void propose_tree_kernel(const int32_t* __restrict__ tokens, int cap,
                                                                   int32_t* __restrict__ state, int nmax, int K,
                                                                   int branches, int depth,
                                                                   int32_t* __restrict__ parents_out,
                                                                   int32_t* __restrict__ drafts_out) {
    __shared__ __attribute__((aligned(16))) int32_t tk[kTreeIds + 8];    // + group reads past the end
    __shared__ unsigned long long keys[kMaxBranches + 1];
    __shared__ unsigned long long wkeys[kMaxBranches * (kTreeThreads / kWave)];
    int len = state[SV_STATE_LEN];
    const bool gated = state[SV_STATE_GATED] != 0;
    if (len < 0 || len > cap) {
        if (threadIdx.x == 0) state[SV_STATE_FLAGS] |= SV_FLAG_CAPACITY;
        len = 0;
    }
    const int32_t* st = tokens;
    const bool in_lds = len <= kTreeIds;
    if (in_lds) {
        stage_ids(tokens, len, tk);
        __syncthreads();
        st = tk;
    }
    propose_tree_block(st, in_lds, len, nmax, K, branches, depth, parents_out, drafts_out, state, gated, keys, wkeys);
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
