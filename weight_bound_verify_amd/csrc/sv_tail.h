// Round-tail device functions shared by the standalone accept / propose kernels and by the
// last workgroup of a fused round (argmax -> accept -> next drafts in one launch).
#pragma once

#include "sv_device.h"

#include <climits>
#include "../../include/specverify.h"

namespace sv {

constexpr int kHalo = SV_MAX_NGRAM;   // ids before an LDS chunk that a match may reach back to

// Copy src[0 .. n) to LDS dst[0 .. n) with the whole workgroup, several 16-byte loads in
// flight per thread (a strided one-id-per-iteration loop would wait on every load).  Ids
// src[i] with i outside [0, n) are never read.  The 16-byte vector path is taken only when
// both `src` and `dst` are 16-byte aligned; otherwise single ids are copied.
__device__ __forceinline__ void stage_ids(const int32_t* __restrict__ src, int n, int32_t* dst) {
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    const int tid = threadIdx.x, nt = blockDim.x;
    int done = 0;
    if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0) {
        const int n4 = n >> 2;
        const i32x4* s4 = reinterpret_cast<const i32x4*>(src);
        i32x4* d4 = reinterpret_cast<i32x4*>(dst);
        constexpr int U = 4;
        for (int base = 0; base < n4; base += nt * U) {
            i32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = base + u * nt + tid;
                if (i < n4) v[u] = s4[i];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = base + u * nt + tid;
                if (i < n4) d4[i] = v[u];
            }
        }
        done = n4 << 2;
    }
    for (int i = done + tid; i < n; i += nt) dst[i] = src[i];
}

// The first n ids of a 16-byte aligned stream held in registers by a whole workgroup (n <=
// 4 NP ids per thread): thread t holds 16-byte pieces t, t + nt, ..., t + (NP-1) nt.  Loading
// them does not depend on the stream length, so a round tail issues these loads together with
// its other independent loads and stores them to LDS afterwards.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
template <int NP>
struct IdPrefix { i32x4_t v[NP]; };

template <int NP>
__device__ __forceinline__ void prefix_load(const int32_t* __restrict__ src, int n, IdPrefix<NP>& p) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const int n4 = n >> 2;
    const i32x4_t* s4 = reinterpret_cast<const i32x4_t*>(src);
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int i = u * nt + tid;
        p.v[u] = i < n4 ? s4[i] : i32x4_t{0, 0, 0, 0};
    }
}

// Ids [lo, n) of a 16-byte aligned stream (lo a multiple of 4 * blockDim.x), in the layout of
// prefix_load over [lo, lo + 4 NP blockDim.x): piece u of thread t holds ids lo + 4 (u nt + t).
template <int NP>
__device__ __forceinline__ void prefix_load_from(const int32_t* __restrict__ src, int lo, int n, IdPrefix<NP>& p) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const int n4 = n >> 2, lo4 = lo >> 2;
    const i32x4_t* s4 = reinterpret_cast<const i32x4_t*>(src);
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int i = lo4 + u * nt + tid;
        p.v[u] = i < n4 ? s4[i] : i32x4_t{0, 0, 0, 0};
    }
}

template <int NP>
__device__ __forceinline__ void prefix_store_from(const int32_t* __restrict__ src, int lo, int n,
                                                  const IdPrefix<NP>& p, int32_t* dst) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const int n4 = n >> 2, lo4 = lo >> 2;
    i32x4_t* d4 = reinterpret_cast<i32x4_t*>(dst);
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int i = lo4 + u * nt + tid;
        if (i < n4) d4[i] = p.v[u];
    }
}

template <int NP>
__device__ __forceinline__ void prefix_store(const int32_t* __restrict__ src, int n, const IdPrefix<NP>& p,
                                             int32_t* dst) {
    const int tid = threadIdx.x, nt = blockDim.x;
    const int n4 = n >> 2;
    i32x4_t* d4 = reinterpret_cast<i32x4_t*>(dst);
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int i = u * nt + tid;
        if (i < n4) d4[i] = p.v[u];
    }
    for (int i = (n4 << 2) + tid; i < n; i += nt) dst[i] = src[i];
}

// Best (match length << 32 | end position) over the end positions e < len - 1 of a stream held
// in LDS (`tk`, 16-byte aligned, at least len ids and readable up to the next multiple of four
// past len - 1), for the share of thread `tid` of `nthreads`: groups of four consecutive end
// positions, group index = tid + k * nthreads.  A group reads its four ids and the NM ids
// before it as 16-byte LDS reads and finds every match from registers (NM = 4 covers nmax <= 4,
// NM = 8 the rest), so the scan costs a few instructions per position.  A position before the
// stream start never matches (its position, not its value, rules it out), and the read index
// is clamped at zero so no read leaves the array.  Host-callable so that its index arithmetic
// can be checked on the CPU.
template <int NM>
__host__ __device__ __forceinline__ unsigned long long scan_best_lds(const int32_t* tk, int len, int nmax,
                                                                     const int32_t (&suf)[SV_MAX_NGRAM], int tid,
                                                                     int nthreads) {
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    const i32x4* t4 = reinterpret_cast<const i32x4*>(tk);
    unsigned long long best = 0;
    const int ngroups = (len - 1 + 3) >> 2;                   // groups holding end positions 0 .. len-2
    for (int gi = tid; gi < ngroups; gi += nthreads) {
        const int e0 = gi << 2;
        int32_t w[NM + 4];                                      // ids e0 - NM .. e0 + 3
#pragma unroll
        for (int q = 0; q < NM / 4 + 1; ++q) {
            // the index is clamped so every read stays inside the array: the compiler merges
            // neighbouring groups' reads into one base and offsets and issues them
            // unconditionally, and a read below the array through a generic pointer would leave
            // the LDS window; what a clamped read returns is never compared (see below)
            const int vi = gi - NM / 4 + q;
            const i32x4 v = t4[vi < 0 ? 0 : vi];
#pragma unroll
            for (int c = 0; c < 4; ++c) w[4 * q + c] = v[c];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + j;
            int l = 0;
            bool run = true;
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                // position e - i = e0 + (j - i) lies before the stream only when i > j and e0 < i - j
                run = run && i < nmax && (i <= j || e0 >= i - j) && w[NM + j - i] == suf[i];
                l += run ? 1 : 0;
            }
            if (l > 0 && e < len - 1) {
                const unsigned long long key = ((unsigned long long)l << 32) | (unsigned)e;
                best = key > best ? key : best;
            }
        }
    }
    return best;
}

constexpr int kMaxBranches = 4;                // branches of the tree drafter

// Insert key k into a descending list of kMaxBranches keys (keys are distinct).
__host__ __device__ __forceinline__ void top_insert(unsigned long long (&top)[kMaxBranches], unsigned long long k) {
#pragma unroll
    for (int b = 0; b < kMaxBranches; ++b)
        if (k > top[b]) { const unsigned long long t = top[b]; top[b] = k; k = t; }
}

// The four best keys (l << 32 | e) of thread `tid` of `nthreads` over the end positions
// e < len - 1 of a stream in LDS (`tk`, 16-byte aligned, readable up to the next multiple of
// four past len - 1): groups of four end positions from 16-byte reads, as the linear
// drafter's scan (NM = 4 covers nmax <= 4, NM = 8 the rest).  A position before the stream
// start never matches (its position rules it out), and the read index is clamped at zero so
// no read leaves the array (the compiler issues neighbouring groups' reads unconditionally
// from one base, and through a generic pointer a read below the array would leave the LDS
// window).  Host-callable so that its index arithmetic can be checked on the CPU.
template <int NM>
__host__ __device__ __forceinline__ void scan_top_lds(const int32_t* tk, int len, int nmax,
                                                      const int32_t (&suf)[SV_MAX_NGRAM],
                                                      unsigned long long (&top)[kMaxBranches], int tid,
                                                      int nthreads) {
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    const i32x4* t4 = reinterpret_cast<const i32x4*>(tk);
    const int ngroups = (len - 1 + 3) >> 2;
    for (int gi = tid; gi < ngroups; gi += nthreads) {
        const int e0 = gi << 2;
        int32_t w[NM + 4];
#pragma unroll
        for (int q = 0; q < NM / 4 + 1; ++q) {
            const int vi = gi - NM / 4 + q;
            const i32x4 v = t4[vi < 0 ? 0 : vi];
#pragma unroll
            for (int c = 0; c < 4; ++c) w[4 * q + c] = v[c];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + j;
            int l = 0;
            bool run = true;
#pragma unroll
            for (int i = 0; i < NM; ++i) {
                run = run && i < nmax && (i <= j || e0 >= i - j) && w[NM + j - i] == suf[i];
                l += run ? 1 : 0;
            }
            if (l > 0 && e < len - 1) top_insert(top, ((unsigned long long)l << 32) | (unsigned)e);
        }
    }
}

// Per-round statistics and the hit-rate gate ("Stream C - Speculative decoding", the shipped
// app note: the drafter is dropped after gateAfter rounds that accepted nothing).  One thread.
__device__ __forceinline__ void record_round(int32_t* state, int j) {
    state[SV_STATE_J] = j;
    const int rounds = state[SV_STATE_ROUNDS] + 1;
    state[SV_STATE_ROUNDS] = rounds;
    state[SV_STATE_SUMJ] += j;
    state[SV_STATE_HIST + j] += 1;
    const int zero_run = j == 0 ? state[SV_STATE_ZERO_RUN] + 1 : 0;
    state[SV_STATE_ZERO_RUN] = zero_run;
    const int gate_after = state[SV_STATE_GATE_AFTER];
    if (gate_after > 0 && state[SV_STATE_GATED] == 0 && zero_run >= gate_after) state[SV_STATE_GATED] = rounds;
}

// The round state's words held by one wave (lane l: state[l] and state[64 + l]), loaded at the
// start of a round tail together with its other loads, so recording the round needs no
// read-modify-write round trip to memory after the accept.
struct StateCache { int32_t lo, hi; };

__device__ __forceinline__ StateCache state_cache_load(const int32_t* state, int lane) {
    StateCache c;
    c.lo = state[lane];
    c.hi = lane < SV_STATE_WORDS - 64 ? state[64 + lane] : 0;
    return c;
}

__device__ __forceinline__ int state_word(const StateCache& c, int idx) {      // idx uniform
    return idx < 64 ? __builtin_amdgcn_readlane(c.lo, idx) : __builtin_amdgcn_readlane(c.hi, idx - 64);
}

// record_round from the cached words, by the whole wave (same updates, same order of rules).
// Returns the gate word after the round.
__device__ __forceinline__ int record_round_cached(const StateCache& c, int32_t* state, int j, int lane) {
    const int rounds = state_word(c, SV_STATE_ROUNDS) + 1;
    const int sumj = state_word(c, SV_STATE_SUMJ) + j;
    const int hist = state_word(c, SV_STATE_HIST + j) + 1;
    const int zero_run = j == 0 ? state_word(c, SV_STATE_ZERO_RUN) + 1 : 0;
    const int gate_after = state_word(c, SV_STATE_GATE_AFTER);
    int gated = state_word(c, SV_STATE_GATED);
    if (gate_after > 0 && gated == 0 && zero_run >= gate_after) gated = rounds;
    if (lane == 0) {
        state[SV_STATE_J] = j;
        state[SV_STATE_ROUNDS] = rounds;
        state[SV_STATE_SUMJ] = sumj;
        state[SV_STATE_HIST + j] = hist;
        state[SV_STATE_ZERO_RUN] = zero_run;
        state[SV_STATE_GATED] = gated;
    }
    return gated;
}

// The drafter's output once the hit-rate gate has fired: K pads, nothing matched.
__device__ __forceinline__ void gated_drafts(int K, int32_t* drafts, int32_t* state) {
    if (threadIdx.x < K) drafts[threadIdx.x] = -1;
    if (threadIdx.x == 0) {
        state[SV_STATE_NVALID] = 0;
        state[SV_STATE_NUSED] = 0;
    }
}

// Argmax stage 2 leaves INT_MAX when no logit of a row compared greater than -inf (every
// logit NaN, e.g. after an overflowed activation); such a row has no greedy id and is
// reported as -1.
__device__ __forceinline__ int argmax_id(int bi) { return bi == INT_MAX ? -1 : bi; }

// Greedy accept by one wave ("Stream C - Speculative decoding", the delta and control-logic
// proof; "Spec-decode on GDN hybrids", hybrid state discipline): lane i compares d_{i+1}
// with the greedy id of window row i, a ballot finds the first miss j, the accepted drafts
// and argmax[j] (correction or bonus) are appended and len advances by 1 + j.  A call that
// could overflow `cap` writes no token and sets the sticky capacity flag; a call whose
// argmax[j] is -1 (that row had no greedy id) writes no token, records no round and sets the
// sticky argmax flag.
__device__ __forceinline__ void accept_wave(const int32_t* argmax, const int32_t* drafts, int K, int32_t* tokens,
                                            int cap, int32_t* state, int lane) {
    const int len = state[SV_STATE_LEN];
    if (len + K + 1 > cap || len < 0) {
        if (lane == 0) state[SV_STATE_FLAGS] |= SV_FLAG_CAPACITY;
        return;
    }
    int d = -1, a = -2;
    if (lane < K) { d = drafts[lane]; a = argmax[lane]; }
    const unsigned long long hit = __ballot(lane < K && d >= 0 && d == a);
    const int j = __builtin_ctzll(~hit);                 // <= K: bit K is never set
    const int aj = argmax[j];                            // the correction or bonus id (uniform)
    if (aj < 0) {
        if (lane == 0) state[SV_STATE_FLAGS] |= SV_FLAG_ARGMAX;
        return;
    }
    if (lane < j) tokens[len + lane] = d;
    if (lane == j) tokens[len + j] = aj;
    if (lane == 0) {
        state[SV_STATE_LEN] = len + 1 + j;
        if (K > 0) record_round(state, j);        // K = 0 is the anchor bootstrap, not a round
    }
}

// Sampling accept by one wave (speculative sampling with a point-mass drafter; "Stream C -
// Speculative decoding", the deferred list: probabilities and a residual redraw instead of an
// argmax comparison).  Lane s < K keeps draft d_{s+1} iff it is a vocabulary id and
// u_s < p_s(d) = exp(zd[s] - lse[s]), u_s the accept uniform of the round (Philox4x32-10
// counter (0, len, s / 4, 1), word s % 4).  j = the first draft not kept; d_1..d_j and row j's
// draw (its residual draw, or the bonus draw when j = K) are appended, so len advances by
// 1 + j.  `mirror` (may be null) receives the same ids at the same positions.  A call that
// could overflow `cap` writes no token and sets the sticky capacity flag.  Returns j, or -1.
// The lane's draft `d` and its scaled logit `zdl` come in registers (lanes >= K: ignored).
__device__ __forceinline__ int accept_sample_regs(const int32_t* sample, const float* lse, int d, float zdl, int K,
                                                  int V, uint32_t key0, uint32_t key1, int32_t* tokens, int cap,
                                                  int32_t* state, int lane, int32_t* mirror,
                                                  const StateCache* cache = nullptr) {
    const int len = cache ? state_word(*cache, SV_STATE_LEN) : state[SV_STATE_LEN];
    if (len + K + 1 > cap || len < 0) {
        if (lane == 0) state[SV_STATE_FLAGS] |= SV_FLAG_CAPACITY;
        return -1;
    }
    if (lane >= K) d = -1;
    bool keep = false;
    if (lane < K && d >= 0 && d < V) {
        const Philox4 rnd = philox4x32_10(0u, (uint32_t)len, (uint32_t)(lane >> 2), 1u, key0, key1);
        const float u = uniform01(philox_word(rnd, lane & 3));
        keep = u < __expf(zdl - lse[lane]);
    }
    const unsigned long long kept = __ballot(keep);
    const int j = __builtin_ctzll(~kept);                // <= K: bit K is never set
    if (sample[j] < 0) {                                 // row j drew nothing (every key NaN)
        if (lane == 0) state[SV_STATE_FLAGS] |= SV_FLAG_ARGMAX;
        return -1;
    }
    if (lane < j) {
        tokens[len + lane] = d;
        if (mirror) mirror[len + lane] = d;
    }
    if (lane == j) {
        tokens[len + j] = sample[j];
        if (mirror) mirror[len + j] = sample[j];
    }
    if (cache) {
        if (lane == 0) state[SV_STATE_LEN] = len + 1 + j;
        if (K > 0) record_round_cached(*cache, state, j, lane);      // K = 0 is the bootstrap, not a round
    } else if (lane == 0) {
        state[SV_STATE_LEN] = len + 1 + j;
        if (K > 0) record_round(state, j);        // K = 0 is the anchor bootstrap, not a round
    }
    return j;
}

// The same accept with the drafts and their scaled logits read from `drafts` / `zd`.
__device__ __forceinline__ int accept_sample_wave(const int32_t* sample, const float* lse, const float* zd,
                                                  const int32_t* drafts, int K, int V, uint32_t key0,
                                                  uint32_t key1, int32_t* tokens, int cap, int32_t* state,
                                                  int lane, int32_t* mirror) {
    int d = -1;
    float zdl = 0.f;
    if (lane < K) {
        d = drafts[lane];
        zdl = zd[lane];
    }
    return accept_sample_regs(sample, lse, d, zdl, K, V, key0, key1, tokens, cap, state, lane, mirror);
}

// n-gram prompt lookup by a whole workgroup ("Stream C - Speculative decoding", the delta:
// One chunk of the global-memory drafter: end positions [base, end) are scanned, and stream
// ids [lo, hi) are staged at tk[dst .. dst + hi - lo) (tk[t] holds id base - kHalo + t).
// Every id a scan of this chunk compares, e - i for e in [base, end), i < nmax <= kHalo and
// e - i >= 0, lies in [lo, hi), and every tk index lies in [0, kHalo + chunk).
struct ChunkWindow {
    int lo, hi, dst, end;
};
__host__ __device__ __forceinline__ ChunkWindow chunk_window(int base, int chunk, int len) {
    ChunkWindow w;
    w.lo = base - kHalo < 0 ? 0 : base - kHalo;
    w.hi = base + chunk < len ? base + chunk : len;
    w.dst = w.lo - (base - kHalo);
    w.end = base + chunk < len - 1 ? base + chunk : len - 1;
    return w;
}

// The (match length, end position) key of end position e against the suffix suf (nmax ids,
// newest first), read from a chunk staged as chunk_window describes: 0 when nothing matches.
__host__ __device__ __forceinline__ unsigned long long chunk_key(const int32_t* tk, int base, int e,
                                                                 const int32_t* suf, int nmax) {
    int l = 0;
#pragma unroll
    for (int i = 0; i < SV_MAX_NGRAM; ++i) {
        if (l == i && i < nmax && e - i >= 0 && tk[e - i - base + kHalo] == suf[i]) l = i + 1;
    }
    return l > 0 ? ((unsigned long long)l << 32) | (unsigned)e : 0ull;
}

// the last m ids of the stream index their most recent continuation; "Spec-decode on GDN
// hybrids", harness lessons: the stream ends in the pending anchor, so drafts continue past
// it).  For every end position e <= len-2 a thread computes the match length l(e) of the
// stream's suffix ending at e (capped at nmax).  "First n from nmax down with a match, latest
// occurrence" is the lexicographic maximum of (l(e), e): one 64-bit max-reduction.  The
// stream is staged through LDS (`tk`, chunk + kHalo ids) so the scan reads HBM once.
// `wbest` holds one slot per wave.  Every thread of the workgroup must call it.
__device__ __forceinline__ void propose_block(const int32_t* tokens, int cap, int32_t* state, int nmax, int K,
                                              int32_t* drafts, int32_t* tk, int chunk,
                                              unsigned long long* wbest) {
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    if (state[SV_STATE_GATED] != 0) {        // the hit-rate gate dropped the drafter
        gated_drafts(K, drafts, state);
        return;
    }
    int len = state[SV_STATE_LEN];
    if (len < 0 || len > cap) {              // corrupt state: never read past the buffer
        if (tid == 0) state[SV_STATE_FLAGS] |= SV_FLAG_CAPACITY;
        len = 0;
    }

    int32_t suf[SV_MAX_NGRAM];
#pragma unroll
    for (int i = 0; i < SV_MAX_NGRAM; ++i) suf[i] = (i < nmax && len - 1 - i >= 0) ? tokens[len - 1 - i] : -1;

    unsigned long long best = 0;
    for (int base = 0; base < len - 1; base += chunk) {
        barrier_lds();
        // ids before the stream start are never staged or compared
        const ChunkWindow w = chunk_window(base, chunk, len);
        stage_ids(tokens + w.lo, w.hi - w.lo, tk + w.dst);
        barrier_lds();
        for (int e = base + tid; e < w.end; e += nthreads) {
            const unsigned long long key = chunk_key(tk, base, e, suf, nmax);
            best = key > best ? key : best;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const unsigned long long o = __shfl_xor(best, off, 64);
        best = o > best ? o : best;
    }
    if ((tid & 63) == 0) wbest[tid >> 6] = best;
    barrier_lds();
    if (tid < kWave) {
        unsigned long long b = tid < nthreads / kWave ? wbest[tid] : 0ull;
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
            state[SV_STATE_NVALID] = nused > 0 ? min(K, len - 1 - e) : 0;
            state[SV_STATE_NUSED] = nused;
        }
    }
}

// Drafter over a stream held whole in LDS (`tk[0 .. len)`, len <= 65536): the same rule as
// propose_block, with no global reads.  End positions fit in 16 bits here, so the key
// (match length, end position) is packed as l << 16 | e and reduced as 32 bits with DPP.  Every
// thread of the workgroup must call it.
__device__ __forceinline__ void propose_lds(const int32_t* tk, int len, int nmax, int K, int32_t* drafts,
                                            int32_t* state, unsigned long long* wbest, bool gated) {
    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    if (gated) {                             // the hit-rate gate dropped the drafter (uniform)
        gated_drafts(K, drafts, state);
        return;
    }
    int32_t suf[SV_MAX_NGRAM];
#pragma unroll
    for (int i = 0; i < SV_MAX_NGRAM; ++i) suf[i] = (i < nmax && len - 1 - i >= 0) ? tk[len - 1 - i] : -1;
    const unsigned long long b64 = nmax <= 4 ? scan_best_lds<4>(tk, len, nmax, suf, tid, nthreads)
                                             : scan_best_lds<8>(tk, len, nmax, suf, tid, nthreads);
    uint32_t best = (uint32_t)((b64 >> 32) << 16) | (uint32_t)(b64 & 0xffffu);
    best = wave_max_u32(best);
    uint32_t* wb = reinterpret_cast<uint32_t*>(wbest);
    if ((tid & 63) == 0) wb[tid >> 6] = best;
    barrier_lds();
    if (tid < kWave) {
        const uint32_t b = wave_max_u32(tid < nthreads / kWave ? wb[tid] : 0u);
        const int nused = (int)(b >> 16);
        const int e = (int)(b & 0xffffu);
        if (tid < K) {
            const int p = e + 1 + tid;
            drafts[tid] = (nused > 0 && p <= len - 1) ? tk[p] : -1;
        }
        if (tid == 0) {
            state[SV_STATE_NVALID] = nused > 0 ? min(K, len - 1 - e) : 0;
            state[SV_STATE_NUSED] = nused;
        }
    }
}

}  // namespace sv
