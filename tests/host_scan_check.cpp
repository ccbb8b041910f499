// Host harness for the round tails' LDS scans (scan_best_lds, scan_top_lds): runs their index
// arithmetic on the CPU, for every simulated thread of a workgroup, over a stream held in a heap
// array of exactly the length the kernels guarantee readable (ids up to the next multiple of
// four past len - 1).  Built with AddressSanitizer, so any read below or past that array (the
// kind of read that faulted the tree drafter's LDS scan on the GPU) stops the run.
//
// It also runs the global-memory drafter's chunked scan (chunk_window, chunk_key) at several
// chunk sizes: each chunk is staged into a heap array of exactly kHalo + chunk ids, whose
// slots outside the staged window hold the suffix's own ids, so a read of an unstaged slot
// would show as a spurious match.
//
// stdin:  cases, then per case: len nmax nthreads, then len ids
// stdout: per case: l e (best of scan_best_lds; 0 0 when nothing matched), then the four best
//         keys of scan_top_lds merged over the threads, as l e pairs (0 0 past the last), then
//         the best key of the chunked scan for each chunk size of kChunks, as l e pairs
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../weight_bound_verify_amd/csrc/sv_tail.h"

static const int kChunks[] = {1, 2, 3, 5, 8, 17, 64, 8192};

// propose_block's scan, chunk by chunk, thread by simulated thread
static unsigned long long chunked_best(const std::vector<int32_t>& ids, int len, int nmax, const int32_t* suf,
                                       int chunk, int nthreads) {
    unsigned long long best = 0;
    const size_t n = (size_t)sv::kHalo + (size_t)chunk;
    for (int base = 0; base < len - 1; base += chunk) {
        int32_t* tk = static_cast<int32_t*>(std::malloc(n * 4));
        if (!tk) std::exit(3);
        for (size_t i = 0; i < n; ++i) tk[i] = suf[i % (nmax > 0 ? nmax : 1)];
        const sv::ChunkWindow w = sv::chunk_window(base, chunk, len);
        if (w.hi > w.lo) std::memcpy(tk + w.dst, ids.data() + w.lo, (size_t)(w.hi - w.lo) * 4);
        // the staged ids stay in place; poison only marks what was never staged
        for (int t = 0; t < nthreads; ++t)
            for (int e = base + t; e < w.end; e += nthreads) {
                const unsigned long long k = sv::chunk_key(tk, base, e, suf, nmax);
                best = k > best ? k : best;
            }
        std::free(tk);
    }
    return best;
}

int main() {
    int cases = 0;
    if (std::scanf("%d", &cases) != 1) return 2;
    for (int c = 0; c < cases; ++c) {
        int len = 0, nmax = 0, nthreads = 0;
        if (std::scanf("%d %d %d", &len, &nmax, &nthreads) != 3) return 2;
        std::vector<int32_t> ids(len);
        for (int i = 0; i < len; ++i)
            if (std::scanf("%d", &ids[i]) != 1) return 2;
        // readable extent: groups cover end positions 0 .. len-2, four per group
        const int ngroups = (len - 1 + 3) >> 2;
        const int extent = ngroups > 0 ? 4 * ngroups : 0;
        const size_t bytes = (size_t)(extent > len ? extent : len) * 4;
        int32_t* tk = static_cast<int32_t*>(std::aligned_alloc(16, bytes > 0 ? (bytes + 15) / 16 * 16 : 16));
        if (!tk) return 3;
        if (len > 0) std::memcpy(tk, ids.data(), (size_t)len * 4);
        // ids past the stream repeat its last id: a scan that compared them would find matches
        for (int i = len; i < (int)(bytes / 4); ++i) tk[i] = len > 0 ? ids[len - 1] : 0;
        int32_t suf[SV_MAX_NGRAM];
        for (int i = 0; i < SV_MAX_NGRAM; ++i) suf[i] = (i < nmax && len - 1 - i >= 0) ? tk[len - 1 - i] : -1;
        unsigned long long best = 0;
        std::vector<unsigned long long> keys;
        for (int t = 0; t < nthreads; ++t) {
            const unsigned long long b = nmax <= 4 ? sv::scan_best_lds<4>(tk, len, nmax, suf, t, nthreads)
                                                   : sv::scan_best_lds<8>(tk, len, nmax, suf, t, nthreads);
            best = b > best ? b : best;
            unsigned long long top[sv::kMaxBranches] = {0ull, 0ull, 0ull, 0ull};
            if (nmax <= 4) sv::scan_top_lds<4>(tk, len, nmax, suf, top, t, nthreads);
            else sv::scan_top_lds<8>(tk, len, nmax, suf, top, t, nthreads);
            for (unsigned long long k : top)
                if (k) keys.push_back(k);
        }
        std::sort(keys.begin(), keys.end(), [](unsigned long long a, unsigned long long b) { return a > b; });
        keys.resize(sv::kMaxBranches, 0ull);
        std::printf("%llu %llu", best >> 32, best & 0xffffffffull);
        for (unsigned long long k : keys) std::printf(" %llu %llu", k >> 32, k & 0xffffffffull);
        for (int chunk : kChunks) {
            const unsigned long long cb = chunked_best(ids, len, nmax, suf, chunk, nthreads < 64 ? nthreads : 64);
            std::printf(" %llu %llu", cb >> 32, cb & 0xffffffffull);
        }
        std::printf("\n");
        std::free(tk);
    }
    return 0;
}
